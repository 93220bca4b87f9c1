// paged_attn_decode_noalloc: the decode with its split-context scratch in a
// buffer of the library's own, for callers that cannot allocate.
//
// The buffer is a file-scope device array, one copy per GPU the library
// runs on, held until the process ends.  In host code its name is only a
// host-side stand-in, so its device address is looked up with
// hipGetSymbolAddress, once per device (with that device current), and that
// address is what the kernels get.

#include "../../include/paged_kv.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "decode.h"

static __device__ __align__(256) char scratch[PAGED_KV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_ptr[kMaxDevices];

}  // namespace

namespace pkv {

void *noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // two threads racing on a device's first call store the same address
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace pkv

extern "C" int paged_attn_decode_noalloc(
    const void *query, const void *key_cache, const void *value_cache,
    const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int num_blocks, int max_blocks_per_seq, int max_context_len, int partition_size, int dtype,
    void *stream) {
    return pkv::run_decode(query, nullptr, nullptr, nullptr, key_cache, value_cache, block_tables,
                           context_lens, scale, out, num_seqs, num_q_heads, num_kv_heads,
                           head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                           partition_size, dtype, nullptr, 0, stream, true);
}

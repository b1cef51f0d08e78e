// Final-stream rows and Cyclic Replication Initialization
// (hd_final_stream_rows, hd_cyclic_replicate).
//
// "Hidden Decoding at Scale" review, section Method: the next-token loss is
// taken only at the final stream's positions (the first n-1 streams are
// latent computation), so the LM head reads the rows p(t, n-1) = t*n + n-1 of
// the expanded sequence; and the expansion factor grows 1 -> 2 -> 4 -> 8 with
// Cyclic Replication Initialization, which fills the new embedding tables with
// copies of the existing ones (new table s = old table s mod n_old).
//
// Both are HBM-bound row copies.  One kernel walks the destination in 16-byte
// chunks (coalesced stores, whole 16-byte pieces of each source row), one
// chunk per thread, with nontemporal loads and stores (the data is touched
// once: keeping it out of the caches measured 12% faster than cached
// accesses with four chunks per thread, 6.5 vs 5.7 TB/s on 2.5 GB); the source
// row of each destination row is the only difference between the two
// operations.
#include "common.h"

namespace hdsfa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 1;

// FINAL: destination row r = b*L + t reads source row b*n*L + t*n + n-1
//        (a = L, b = n).
// CYCLIC: blockIdx.y = destination table s0 + y, which reads table
//        (s0 + y) mod n_old; chunks index the table (a = s0, b = n_old).
template <bool FINAL>
__global__ void __launch_bounds__(kCopyThreads)
rowcopy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
               uint32_t chunks, uint32_t cpr, uint32_t a, uint32_t b) {
    const uint32_t base = blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
    const u32x4* s;
    u32x4* d;
    if constexpr (FINAL) {
        s = src;
        d = dst;
    } else {
        const uint32_t t = a + blockIdx.y;
        s = src + (uint64_t)(t % b) * chunks;
        d = dst + (uint64_t)t * chunks;
    }
    u32x4 val[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t c = base + (uint32_t)u * kCopyThreads;
        if (c < chunks) {
            if constexpr (FINAL) {
                const uint32_t r = c / cpr;
                const uint32_t w = c - r * cpr;
                const uint32_t bb = r / a;
                const uint32_t t = r - bb * a;
                const uint64_t srow = ((uint64_t)bb * a + t) * b + (b - 1);
                val[u] = __builtin_nontemporal_load(s + srow * cpr + w);
            } else {
                val[u] = __builtin_nontemporal_load(s + c);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t c = base + (uint32_t)u * kCopyThreads;
        if (c < chunks) __builtin_nontemporal_store(val[u], d + c);
    }
}

bool overlap(const void* p, uint64_t pb, const void* q, uint64_t qb) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), c = reinterpret_cast<uintptr_t>(q);
    return a < c + qb && c < a + pb;
}

}  // namespace

}  // namespace hdsfa

extern "C" hd_status hd_final_stream_rows(const uint16_t* x, int64_t B, int32_t n, int64_t L,
                                          int64_t H, uint16_t* out, hipStream_t stream) {
    using namespace hdsfa;
    if (B < 0 || L < 0 || n < 1 || H <= 0 || H % 8 != 0) return HD_ERR_SHAPE;
    if (B == 0 || L == 0) return HD_OK;
    if (x == nullptr || out == nullptr) return HD_ERR_NULL;
    if (!aligned16(x) || !aligned16(out)) return HD_ERR_SHAPE;
    const uint64_t cpr = (uint64_t)H / 8;
    const uint64_t chunks = (uint64_t)B * (uint64_t)L * cpr;
    if (chunks >= 0xffffffffULL || (uint64_t)L >= 0xffffffffULL || cpr >= 0xffffffffULL)
        return HD_ERR_UNSUPPORTED;
    if (overlap(x, (uint64_t)B * n * L * H * 2, out, chunks * 16)) return HD_ERR_SHAPE;
    const uint64_t per_block = (uint64_t)kCopyThreads * kCopyUnroll;
    const uint32_t blocks = (uint32_t)((chunks + per_block - 1) / per_block);
    rowcopy_kernel<true><<<dim3(blocks), dim3(kCopyThreads), 0, stream>>>(
        reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(out), (uint32_t)chunks,
        (uint32_t)cpr, (uint32_t)L, (uint32_t)n);
    return launch_status();
}

extern "C" hd_status hd_cyclic_replicate(const uint16_t* tables, int32_t n_old, int64_t V,
                                         int64_t H, uint16_t* out, int32_t n_new,
                                         hipStream_t stream) {
    using namespace hdsfa;
    if (n_old < 1 || n_new < 1 || V < 0 || H <= 0 || H % 8 != 0) return HD_ERR_SHAPE;
    if (V == 0) return HD_OK;
    if (tables == nullptr || out == nullptr) return HD_ERR_NULL;
    if (!aligned16(tables) || !aligned16(out)) return HD_ERR_SHAPE;
    const uint64_t chunks = (uint64_t)V * (uint64_t)H / 8;     // per table
    if (chunks >= 0xffffffffULL || n_new > 65535) return HD_ERR_UNSUPPORTED;
    // in place (out == tables): the first n_old tables already hold themselves
    const bool in_place = static_cast<const void*>(out) == static_cast<const void*>(tables);
    if (!in_place && overlap(tables, (uint64_t)n_old * chunks * 16, out, (uint64_t)n_new * chunks * 16))
        return HD_ERR_SHAPE;
    const int32_t s0 = in_place ? n_old : 0;
    if (s0 >= n_new) return HD_OK;
    const uint64_t per_block = (uint64_t)kCopyThreads * kCopyUnroll;
    const uint32_t blocks = (uint32_t)((chunks + per_block - 1) / per_block);
    rowcopy_kernel<false><<<dim3(blocks, (uint32_t)(n_new - s0)), dim3(kCopyThreads), 0, stream>>>(
        reinterpret_cast<const u32x4*>(tables), reinterpret_cast<u32x4*>(out), (uint32_t)chunks,
        0u, (uint32_t)s0, (uint32_t)n_old);
    return launch_status();
}

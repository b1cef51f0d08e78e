// Hidden Decoding embedding expansion + interleave (hd_expand).
//
// "Hidden Decoding at Scale" review, section Method, and the
// Tencent/Sequential-Hidden-Decoding README, section Key Idea (items 1-2):
// every token becomes n streams, stream s taken from its own embedding table,
// laid out as one length-nL sequence.  Position of (t, s) is t*n + s.
//
// HBM-bound gather: each output row is an H-element bf16 row of table s.  The
// kernel walks the output in 16-byte chunks, so stores are fully coalesced and
// every table row is read as whole 16-byte pieces.  Each thread keeps UNROLL
// independent loads in flight before storing.
#include "common.h"

namespace hdsfa {

namespace {

constexpr int kExpandThreads = 256;
constexpr int kExpandUnroll = 4;

__global__ void __launch_bounds__(kExpandThreads)
expand_kernel(const int32_t* __restrict__ ids, const u32x4* __restrict__ tables,
              u32x4* __restrict__ out, int32_t* __restrict__ err_flag,
              uint32_t n, uint32_t V, uint32_t chunks_per_row, uint32_t total_chunks) {
    const uint32_t base = blockIdx.x * (kExpandThreads * kExpandUnroll) + threadIdx.x;
    u32x4 val[kExpandUnroll];
#pragma unroll
    for (int u = 0; u < kExpandUnroll; ++u) {
        const uint32_t c = base + (uint32_t)u * kExpandThreads;
        val[u] = u32x4{0u, 0u, 0u, 0u};
        if (c < total_chunks) {
            // output row r = (b*L + t)*n + s, 16-byte chunk w inside the row
            const uint32_t r = c / chunks_per_row;
            const uint32_t w = c - r * chunks_per_row;
            const uint32_t bt = r / n;
            const uint32_t s = r - bt * n;
            const int32_t tok = ids[bt];
            if (tok >= 0 && (uint32_t)tok < V) {
                val[u] = tables[((uint64_t)s * V + (uint32_t)tok) * chunks_per_row + w];
            } else if (err_flag != nullptr) {
                *err_flag = 1;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kExpandUnroll; ++u) {
        const uint32_t c = base + (uint32_t)u * kExpandThreads;
        if (c < total_chunks) out[c] = val[u];
    }
}

}  // namespace

}  // namespace hdsfa

extern "C" hd_status hd_expand(const int32_t* ids, int64_t B, int64_t L,
                               const uint16_t* tables, int32_t n, int64_t V,
                               int64_t H, uint16_t* out, int32_t* err_flag,
                               hipStream_t stream) {
    using namespace hdsfa;
    if (B < 0 || L < 0 || n < 1 || V < 1 || H < 1) return HD_ERR_SHAPE;
    if (B == 0 || L == 0) return HD_OK;
    if (ids == nullptr || tables == nullptr || out == nullptr) return HD_ERR_NULL;
    if (H % 8 != 0 || !aligned16(tables) || !aligned16(out)) return HD_ERR_SHAPE;
    // 32-bit chunk indices: the output may hold at most 2^32 - 2^10 16-byte chunks
    const uint64_t chunks_per_row = (uint64_t)H / 8;
    const uint64_t total = (uint64_t)B * (uint64_t)L * (uint64_t)n * chunks_per_row;
    const uint64_t per_block = (uint64_t)kExpandThreads * kExpandUnroll;
    if (V > 0xffffffffLL || total > 0xffffffffULL - per_block) return HD_ERR_UNSUPPORTED;
    const uint64_t blocks = (total + per_block - 1) / per_block;
    expand_kernel<<<dim3((uint32_t)blocks), dim3(kExpandThreads), 0, stream>>>(
        ids, reinterpret_cast<const u32x4*>(tables), reinterpret_cast<u32x4*>(out),
        err_flag, (uint32_t)n, (uint32_t)V, (uint32_t)chunks_per_row, (uint32_t)total);
    return launch_status();
}

// Stream-Factorized Attention, prefill (sfa_stream_attn, sfa_mix_attn).
//
// "Hidden Decoding at Scale" review, section Method: most layers attend only
// within their own stream (cost of order n*L^2), a few mix streams with the
// base model's full causal pattern over the length-nL sequence.  The arXiv
// 2607.08186 abstract: this keeps attention cost roughly linear in n.
//
// One kernel serves both layer kinds.  It runs causal attention over a
// strided *view* of the interleaved sequence:
//   within-stream: n views per (batch, KV head), view s = rows s, s+n, s+2n...
//                  of length L (row stride n*H*D elements);
//   mixing:        one view of length nL with row stride H*D.
// In (stream, token) coordinates the within-stream mask is block diagonal over
// streams and lower-triangular over tokens, so a workgroup only ever visits
// key tiles of its own stream that are not in its future: nothing is computed
// for the (n-1)/n of pairs the mask removes.
//
// Workgroup = 4 waves.  Each wave owns 32 query rows of one query head and
// computes S^T = K Q^T and O^T += V^T P^T with the gfx950 bf16 matrix op
// v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  Keeping S transposed puts one
// query per lane (pair of lanes), so row max / row sum are per-lane values
// plus one exchange with the other half-wave, and the probabilities leave the
// accumulator already in the B-operand layout of the second product.
// GQA: the query heads sharing a KV head are packed into one workgroup (up to
// 4, one per wave) so each K/V tile is staged once in LDS for all of them and
// every wave has the same causal extent.
//
// K is staged in LDS row-major with a 16-byte row pad (conflict-free 16-byte
// reads); V is staged transposed ([d][key]) with keys permuted inside each
// 16-key group so that one 16-byte LDS read yields exactly the 8 keys a lane
// needs for the V^T operand.  Tiles are double-buffered in LDS with a
// register prefetch of the next tile, one barrier per tile.
#include "common.h"

namespace hdsfa {

namespace {

constexpr int BN = 64;       // keys per tile
constexpr int MQ = 32;       // query rows per wave
constexpr int NW = 4;        // waves per workgroup
constexpr int THREADS = NW * kWave;
constexpr int VP = BN + 8;   // transposed-V row pitch (elements)

struct PrefillArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    uint64_t q_row;      // elements between consecutive rows of a view (Q, O)
    uint64_t kv_row;     // same for K, V
    uint64_t q_group;    // elements between the first rows of adjacent views
    uint64_t kv_group;
    uint64_t q_batch;    // elements per batch entry
    uint64_t kv_batch;
    uint32_t len;        // rows per view
    uint32_t groups;     // views per (batch, KV head)
    uint32_t B;
    uint32_t Hkv;
    uint32_t G;          // query heads per KV head
    uint32_t P;          // query heads packed per workgroup (1, 2 or 4)
    uint32_t n_hpacks;   // G / P
    uint32_t n_qtiles;   // ceil(len / (MQ * NW / P))
    float c;             // softmax scale * log2(e)
};

// Position, within the transposed-V row, of the first of 4 consecutive keys
// 4*kq .. 4*kq+3 (see the file comment).
__device__ __forceinline__ int vt_pos(int kq) {
    const int qq = kq & 3;
    return 16 * (kq >> 2) + ((qq & 1) << 3) + ((qq >> 1) << 2);
}

template <int D>
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
sfa_prefill_kernel(const PrefillArgs a) {
    constexpr int KP = D + 8;                  // K row pitch (elements)
    constexpr int KS_ELEMS = BN * KP;
    constexpr int VT_ELEMS = D * VP;
    constexpr int BUF_ELEMS = KS_ELEMS + VT_ELEMS;
    constexpr int DSTEPS = D / 16;             // k-steps of the score product
    constexpr int DBLK = D / 32;               // 32-row blocks of O^T
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int K_CHUNKS = BN * CPR / THREADS;        // per thread
    constexpr int V_TASKS = (BN / 4) * (D / 8);         // (key quad, d octet)
    static_assert(BN * CPR % THREADS == 0, "tile/thread mismatch");
    static_assert(V_TASKS <= THREADS, "tile/thread mismatch");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BUF_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;                  // half-wave index

    // ---- work item (longest query tiles first) ----
    uint32_t id = blockIdx.x;
    const uint32_t per_tile = a.B * a.groups * a.Hkv * a.n_hpacks;
    const uint32_t qtile = a.n_qtiles - 1 - id / per_tile;
    id %= per_tile;
    const uint32_t hp = id % a.n_hpacks;
    id /= a.n_hpacks;
    const uint32_t kvh = id % a.Hkv;
    id /= a.Hkv;
    const uint32_t grp = id % a.groups;
    const uint32_t b = id / a.groups;

    const int qblocks = NW / a.P;
    const int BT = MQ * qblocks;               // query rows per workgroup
    const uint32_t head = kvh * a.G + hp * a.P + (wave % a.P);
    const uint32_t q0 = qtile * BT + (wave / a.P) * MQ;

    const uint16_t* qbase = a.q + b * a.q_batch + grp * a.q_group + (uint64_t)head * D;
    uint16_t* obase = a.o + b * a.q_batch + grp * a.q_group + (uint64_t)head * D;
    const uint16_t* kbase = a.k + b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D;
    const uint16_t* vbase = a.v + b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D;

    const uint32_t wg_end = min(a.len, (qtile + 1) * (uint32_t)BT);
    const int n_kt = (int)((wg_end + BN - 1) / BN);
    const uint32_t wave_end = min(a.len, q0 + MQ);       // exclusive
    const int wave_kt = q0 < a.len ? (int)((wave_end + BN - 1) / BN) : 0;

    // ---- Q fragments: lane holds query q0+l32, dims 16e + 8hh .. +7 ----
    const uint32_t qi = q0 + l32;
    bf16x8 qf[DSTEPS];
    {
        const bool ok = qi < a.len;
        const u32x4* src = reinterpret_cast<const u32x4*>(qbase + (uint64_t)qi * a.q_row);
#pragma unroll
        for (int e = 0; e < DSTEPS; ++e) {
            u32x4 w = ok ? src[2 * e + hh] : u32x4{0u, 0u, 0u, 0u};
            qf[e] = __builtin_bit_cast(bf16x8, w);
        }
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;   // running max, in log2 units (already * c)
    float l_run = 0.f;         // running sum of exp2

    // ---- K/V tile staging (global -> registers -> LDS) ----
    u32x4 kreg[K_CHUNKS];
    u32x4 vreg[4];
    const int vkq = tid % (BN / 4);            // key quad of this thread's V task
    const int vdo = tid / (BN / 4);            // d octet
    const bool vtask = tid < V_TASKS;

    auto load_tile = [&](int kt) {
        const uint32_t k0 = (uint32_t)kt * BN;
#pragma unroll
        for (int i = 0; i < K_CHUNKS; ++i) {
            const int cidx = tid + i * THREADS;
            const int row = cidx / CPR;
            const int col = cidx % CPR;
            const uint32_t key = k0 + row;
            kreg[i] = key < a.len
                ? *reinterpret_cast<const u32x4*>(kbase + (uint64_t)key * a.kv_row + col * 8)
                : u32x4{0u, 0u, 0u, 0u};
        }
        if (vtask) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t key = k0 + 4 * vkq + r;
                vreg[r] = key < a.len
                    ? *reinterpret_cast<const u32x4*>(vbase + (uint64_t)key * a.kv_row + vdo * 8)
                    : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* ks = smem + buf * BUF_ELEMS;
        uint16_t* vt = ks + KS_ELEMS;
#pragma unroll
        for (int i = 0; i < K_CHUNKS; ++i) {
            const int cidx = tid + i * THREADS;
            const int row = cidx / CPR;
            const int col = cidx % CPR;
            *reinterpret_cast<u32x4*>(ks + row * KP + col * 8) = kreg[i];
        }
        if (vtask) {
            const int pos = vt_pos(vkq);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int w = j >> 1;
                const int sh = (j & 1) * 16;
                const uint32_t e0 = (vreg[0][w] >> sh) & 0xffffu;
                const uint32_t e1 = (vreg[1][w] >> sh) & 0xffffu;
                const uint32_t e2 = (vreg[2][w] >> sh) & 0xffffu;
                const uint32_t e3 = (vreg[3][w] >> sh) & 0xffffu;
                u32x2 pk = {e0 | (e1 << 16), e2 | (e3 << 16)};
                *reinterpret_cast<u32x2*>(vt + (vdo * 8 + j) * VP + pos) = pk;
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < n_kt; ++kt) {
        if (kt + 1 < n_kt) load_tile(kt + 1);

        if (kt < wave_kt) {
            const uint16_t* ks = smem + (kt & 1) * BUF_ELEMS;
            const uint16_t* vt = ks + KS_ELEMS;

            // S^T[key][query] for two 32-key blocks
            f32x16 sacc[BN / 32];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                sacc[kb] = f32x16{};
                const uint16_t* krow = ks + (kb * 32 + l32) * KP + hh * 8;
#pragma unroll
                for (int e = 0; e < DSTEPS; ++e) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 16 * e);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[e], sacc[kb], 0, 0, 0);
                }
            }

            // causal mask, only where the tile reaches past the wave's first query
            const uint32_t k0 = (uint32_t)kt * BN;
            if (k0 + BN - 1 > q0) {
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                    for (int it = 0; it < 16; ++it) {
                        const uint32_t key = k0 + kb * 32 + 8 * (it >> 2) + 4 * hh + (it & 3);
                        if (key > qi) sacc[kb][it] = -INFINITY;
                    }
            }

            // online softmax (per lane = per query; halves exchange once)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int it = 0; it < 16; ++it) mx = fmaxf(mx, sacc[kb][it]);
            mx = fmaxf(mx, xor32(mx));
            const float m_new = fmaxf(m_run, mx * a.c);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            m_run = m_new;

            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int it = 0; it < 16; ++it) {
                    const float p = fast_exp2(__builtin_fmaf(sacc[kb][it], a.c, -m_use));
                    sacc[kb][it] = p;
                    rs += p;
                }
            rs += xor32(rs);
            l_run = l_run * alpha + rs;
#pragma unroll
            for (int i = 0; i < DBLK; ++i) oacc[i] *= alpha;

            // P^T fragments (B operand): 16-key step c takes items 8*(c%2)..+7
            bf16x8 pf[BN / 16];
#pragma unroll
            for (int c = 0; c < BN / 16; ++c) {
                const f32x16& s = sacc[c >> 1];
                const int o8 = (c & 1) * 8;
                u32x4 w;
                w[0] = pack_bf16x2(s[o8 + 0], s[o8 + 1]);
                w[1] = pack_bf16x2(s[o8 + 2], s[o8 + 3]);
                w[2] = pack_bf16x2(s[o8 + 4], s[o8 + 5]);
                w[3] = pack_bf16x2(s[o8 + 6], s[o8 + 7]);
                pf[c] = __builtin_bit_cast(bf16x8, w);
            }

            // O^T[d][query] += V^T P^T
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const uint16_t* vrow = vt + (db * 32 + l32) * VP + hh * 8;
#pragma unroll
                for (int c = 0; c < BN / 16; ++c) {
                    const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vrow + 16 * c);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], oacc[db], 0, 0, 0);
                }
            }
        }

        if (kt + 1 < n_kt) store_tile((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, lane writes 4 consecutive dims per item group ----
    if (qi < a.len) {
        const float inv = 1.f / l_run;
        uint16_t* orow = obase + (uint64_t)qi * a.q_row;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hh;
                u32x2 w = {pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                           pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + d) = w;
            }
    }
}

hd_status launch_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         uint16_t* out, int64_t B, int32_t n, int64_t L, int32_t Hq,
                         int32_t Hkv, int32_t D, float scale, hipStream_t stream,
                         bool within) {
    if (B < 0 || L < 0 || n < 1 || Hq < 1 || Hkv < 1) return HD_ERR_SHAPE;
    if (Hq % Hkv != 0) return HD_ERR_SHAPE;
    if (D != 64 && D != 128) return HD_ERR_UNSUPPORTED;
    if (B == 0 || L == 0) return HD_OK;
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return HD_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return HD_ERR_SHAPE;
    const int64_t N = (int64_t)n * L;
    if (N > 0x7fffffffLL) return HD_ERR_UNSUPPORTED;

    PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = out;
    const uint64_t row_mult = within ? (uint64_t)n : 1u;
    a.q_row = row_mult * (uint64_t)Hq * D;
    a.kv_row = row_mult * (uint64_t)Hkv * D;
    a.q_group = (uint64_t)Hq * D;
    a.kv_group = (uint64_t)Hkv * D;
    a.q_batch = (uint64_t)N * Hq * D;
    a.kv_batch = (uint64_t)N * Hkv * D;
    a.len = (uint32_t)(within ? L : N);
    a.groups = within ? (uint32_t)n : 1u;
    a.B = (uint32_t)B;
    a.Hkv = (uint32_t)Hkv;
    a.G = (uint32_t)(Hq / Hkv);
    a.P = (a.G % 4 == 0) ? 4u : ((a.G % 2 == 0) ? 2u : 1u);
    a.n_hpacks = a.G / a.P;
    const uint32_t BT = MQ * (NW / a.P);
    a.n_qtiles = (a.len + BT - 1) / BT;
    a.c = scale * kLog2e;

    const uint64_t blocks = (uint64_t)a.n_qtiles * a.B * a.groups * a.Hkv * a.n_hpacks;
    if (blocks > 0x7fffffffULL) return HD_ERR_UNSUPPORTED;
    if (D == 128)
        sfa_prefill_kernel<128><<<dim3((uint32_t)blocks), dim3(THREADS), 0, stream>>>(a);
    else
        sfa_prefill_kernel<64><<<dim3((uint32_t)blocks), dim3(THREADS), 0, stream>>>(a);
    return launch_status();
}

}  // namespace

}  // namespace hdsfa

extern "C" hd_status sfa_stream_attn(const uint16_t* q, const uint16_t* k,
                                     const uint16_t* v, uint16_t* out, int64_t B,
                                     int32_t n, int64_t L, int32_t Hq, int32_t Hkv,
                                     int32_t D, float softmax_scale,
                                     hipStream_t stream) {
    return hdsfa::launch_prefill(q, k, v, out, B, n, L, Hq, Hkv, D, softmax_scale,
                                 stream, /*within=*/true);
}

extern "C" hd_status sfa_mix_attn(const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, uint16_t* out, int64_t B,
                                  int32_t n, int64_t L, int32_t Hq, int32_t Hkv,
                                  int32_t D, float softmax_scale, hipStream_t stream) {
    return hdsfa::launch_prefill(q, k, v, out, B, n, L, Hq, Hkv, D, softmax_scale,
                                 stream, /*within=*/false);
}

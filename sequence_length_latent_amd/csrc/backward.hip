// Stream-Factorized Attention, gradients of a prefill layer (sfa_attn_bwd,
// sfa_attn_bwd_window).
//
// "Hidden Decoding at Scale" review, sections Method and Results: the model
// is trained on the length-nL sequence with the within-stream / mixing
// attention pattern, and the per-batch training cost (5.1x / 4.4x at n=4) is
// the method's price, so the layer's gradient runs on the same strided views
// as the forward (within-stream: n views of length L per (batch, KV head);
// mixing: one view of length nL).  With P the masked softmax of scale * Q K^T,
// lse_i the log-sum-exp of row i (saved by the forward), O = P V and dO the
// upstream gradient:
//
//   dP = dO V^T,   delta_i = sum_j P_ij dP_ij  (= sum_d dO_id O_id)
//   dS = P * (dP - delta)
//   dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO
//
// Two kernels, no atomics (results are bitwise reproducible):
//   dq_kernel     per 64-query tile (the forward's work items): S^T = K Q^T,
//                 P^T from lse, dP^T = V dO^T; a first pass over the key
//                 tiles of the causal range sums delta (stored in the fp32
//                 workspace for dkv_kernel), a second one accumulates
//                 dQ^T += K^T dS^T (one query per lane, K/V tiles staged in
//                 LDS, K^T through transpose reads);
//   dkv_kernel    per 128-key tile (one wave per SIMD, 32 keys per wave):
//                 S = Q K^T, P from lse, dP = dO V^T, dV^T += dO^T P and
//                 dK^T += Q^T dS over every query head of the KV group and the
//                 query tiles at or after the keys (one key per lane, Q / dO
//                 tiles staged in LDS, dO^T and Q^T through transpose reads).
// Sliding-window mixing layers (sfa_attn_bwd_window; the review's Method:
// mixing layers follow the base model's pattern, sliding-window or full):
// query i sees keys i - W < j <= i, so dq_kernel starts at the first key tile
// inside a tile's windows and dkv_kernel stops at the last query tile whose
// windows reach the keys (WIN instances; the masks drop i - j >= W).
// All products are v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulate).
// The gradients sum many unnormalised terms (a key collects dS from every
// later query of every head of its group), so P and dS enter the products as
// a bf16 pair hi + lo (hi = bf16(x), lo = bf16(x - hi)): two MFMAs per
// operand, and the operand rounding drops from 2^-9 to about 2^-17 relative.
#include "common.h"

#include <type_traits>

namespace hdsfa {

namespace {

constexpr int BN = 64;      // rows per staged tile (keys for dq, queries for dkv)
constexpr int MQ = 32;      // rows per wave block
constexpr int NWQ = 8;      // waves per dq workgroup (2 per SIMD)
constexpr int NWK = 4;      // waves per dkv workgroup (1 per SIMD)
constexpr int KV_TILE = MQ * NWK;   // keys per dkv work item

typedef short v4i16 __attribute__((ext_vector_type(4)));

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float* lse;        // [B, Hq, N] natural log
    float* delta;            // [B, Hq, N] workspace
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    uint64_t q_row, kv_row;  // elements between consecutive rows of a view
    uint64_t q_group, kv_group;
    uint64_t q_batch, kv_batch;
    uint32_t len;            // rows per view
    uint32_t groups;         // views per (batch, KV head)
    uint32_t B, Hkv, G, Hq, N;
    uint32_t P, n_hpacks, n_qtiles, n_items;   // dq work items (forward's packing)
    uint32_t n_ktiles, n_kitems;               // dkv work items
    float c;                 // scale * log2(e)
    float scale;
    uint32_t window;         // sliding window W (WIN instances only; W < len)
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds16(const unsigned char* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// x = hi + lo with both halves in bf16 (lo carries the rounding error of hi).
// hi is read back as floats from its packed words (element 2k in the low
// half, 2k + 1 in the high half: a shift and a mask), not converted again.
__device__ __forceinline__ void split_bf16(const f32x8& x, bf16x8& hi, bf16x8& lo) {
    hi = to_bf16x8(x);
    const u32x4 w = __builtin_bit_cast(u32x4, hi);
    f32x8 h;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        h[2 * k] = __builtin_bit_cast(float, w[k] << 16);
        h[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
    }
    lo = to_bf16x8(x - h);
}

// two 8-byte transpose reads -> one A operand
__device__ __forceinline__ bf16x8 lds_tr(const unsigned char* p0, const unsigned char* p1) {
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(p0));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(p1));
    struct { v4i16 x, y; } t{a, b};
    return __builtin_bit_cast(bf16x8, t);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, bool WIN>
__global__ void __launch_bounds__(NWQ * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
dq_kernel(const BwdArgs a) {
    constexpr int ROWB = D * 2;
    constexpr int TILE_B = BN * ROWB;
    constexpr int THREADS = NWQ * kWave;
    constexpr int LOADS = TILE_B / (THREADS * 16);
    constexpr int DSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    static_assert(TILE_B % (THREADS * 16) == 0, "tile/thread mismatch");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TILE_B];   // K x2, V x2

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    // work item: the forward's (query tile, batch, view, KV head, head pack)
    const uint32_t per_tile = a.B * a.groups * a.Hkv * a.n_hpacks;
    uint32_t id = blockIdx.x;
    const uint32_t qtile = a.n_qtiles - 1 - id / per_tile;
    id %= per_tile;
    const uint32_t hp = id % a.n_hpacks;
    id /= a.n_hpacks;
    const uint32_t kvh = id % a.Hkv;
    id /= a.Hkv;
    const uint32_t grp = id % a.groups;
    const uint32_t b = id / a.groups;
    const uint32_t BT = MQ * (NWQ / a.P);
    const uint32_t h = kvh * a.G + hp * a.P + (uint32_t)wave % a.P;
    const uint32_t q0 = qtile * BT + ((uint32_t)wave / a.P) * MQ;
    const uint32_t wg_end = min(a.len, (qtile + 1) * BT);
    const int n_kt = (int)((wg_end + BN - 1) / BN);
    const int last = q0 < a.len ? (int)((min(a.len, q0 + MQ) + BN - 1) / BN) - 1 : -1;
    // first key tile of the workgroup's windows and of this wave's (0 without a window)
    int m_lo = 0, wave_lo = 0;
    if constexpr (WIN) {
        const uint32_t f0 = qtile * BT;
        m_lo = (int)((f0 >= a.window ? f0 - a.window + 1 : 0u) / BN);
        wave_lo = (int)((q0 >= a.window ? q0 - a.window + 1 : 0u) / BN);
    }
    const uint32_t qi = q0 + l32;                       // this lane's query row
    const uint32_t qr = min(qi, a.len - 1u);

    // Q and dO fragments (B operands): lane (l32, hh) holds row qi, dims 16e + 8hh .. +7
    const uint64_t qoff = b * a.q_batch + grp * a.q_group + (uint64_t)h * D + (uint64_t)qr * a.q_row;
    bf16x8 qf[DSTEPS], dof[DSTEPS];
#pragma unroll
    for (int e = 0; e < DSTEPS; ++e) {
        qf[e] = *reinterpret_cast<const bf16x8*>(a.q + qoff + (2 * e + hh) * 8);
        dof[e] = *reinterpret_cast<const bf16x8*>(a.dout + qoff + (2 * e + hh) * 8);
    }
    const uint64_t srow = ((uint64_t)b * a.Hq + h) * a.N + (uint64_t)qr * a.groups + grp;
    const float lse2 = a.lse[srow] * kLog2e;            // log2 units of c * s

    // K / V tile loads (the forward's scheme: row-major, swizzled 16-byte chunks)
    const char* kview = reinterpret_cast<const char*>(a.k + b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D);
    const char* vview = reinterpret_cast<const char*>(a.v + b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D);
    const uint32_t kv_row_b = (uint32_t)a.kv_row * 2u;
    auto issue = [&](const char* view, int kt, unsigned char* buf) {
        const uint32_t k0 = (uint32_t)kt * BN;
        const char* base = view + (uint64_t)k0 * kv_row_b;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const uint32_t lin = (uint32_t)(wave * LOADS + j) * 1024u + (uint32_t)lane * 16u;
            const uint32_t row = lin / ROWB, pch = (lin % ROWB) / 16u;
            const uint32_t srow_ = min(row, a.len - 1u - k0);          // clamp past the view end
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(base + srow_ * kv_row_b + ((pch ^ swz<D>(row)) << 4)),
                (void __attribute__((address_space(3)))*)(buf + (wave * LOADS + j) * 1024), 16, 0, 0);
        }
    };
    auto kbuf = [&](int t) { return smem + (t & 1) * TILE_B; };
    auto vbuf = [&](int t) { return smem + (2 + (t & 1)) * TILE_B; };

    // per-lane LDS offsets: direct reads (row kb*32 + l32, chunk 2e + hh) and
    // transpose reads (the forward's V^T addressing, used here for K^T)
    const uint32_t dsw = swz<D>((uint32_t)l32);
    uint32_t doff[DSTEPS];
#pragma unroll
    for (int e = 0; e < DSTEPS; ++e) doff[e] = (uint32_t)l32 * ROWB + ((((uint32_t)(2 * e + hh)) ^ dsw) << 4);
    const uint32_t vg = (uint32_t)lane >> 4, vr = (uint32_t)lane & 15u;
    const uint32_t vk = vr >> 2, va = vr & 3u;
    uint32_t toff[2][DBLK];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const uint32_t key = 4u * (vg >> 1) + vk + 8u * rd;
        const uint32_t sw = swz<D>(key);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const uint32_t lch = 4u * db + 2u * (vg & 1u) + (va >> 1);
            toff[rd][db] = key * ROWB + ((lch ^ sw) << 4) + (va & 1u) * 8u;
        }
    }

    f32x16 dqt[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) dqt[i] = f32x16{};

    // Two passes over the key tiles of the causal range.  Pass 0 sums
    // delta_i = sum_j P_ij dP_ij (= dO_i . O_i with the exact O, which the
    // bf16-rounded forward output would only approximate); pass 1 forms dS
    // and accumulates dQ^T.
    float dl = 0.f;
    auto pass = [&](auto second) {
        constexpr bool SECOND = decltype(second)::value;
        float dsum[4] = {0.f, 0.f, 0.f, 0.f};
        issue(kview, m_lo, kbuf(m_lo));
        issue(vview, m_lo, vbuf(m_lo));
        for (int m = m_lo; m < n_kt; ++m) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (m + 1 < n_kt) {
                issue(kview, m + 1, kbuf(m + 1));
                issue(vview, m + 1, vbuf(m + 1));
            }
            if (m > last || m < wave_lo) continue;
            const unsigned char* kt = kbuf(m);
            const unsigned char* vt = vbuf(m);
            // S^T = K Q^T and dP^T = V dO^T (64 keys x 32 queries)
            f32x16 st[2] = {f32x16{}, f32x16{}}, dpt[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int e = 0; e < DSTEPS; ++e)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    st[kb] = mfma(lds16(kt + kb * 32 * ROWB + doff[e]), qf[e], st[kb]);
                    dpt[kb] = mfma(lds16(vt + kb * 32 * ROWB + doff[e]), dof[e], dpt[kb]);
                }
            // P^T = 2^(c s - lse2), masked past the query (and before its
            // window).  The masks are applied to the scores (-inf, so P = 0:
            // the scale is positive) and only on the wave's diagonal tile and
            // (WIN) on tiles reaching below some row's window; the other tiles
            // carry no mask work.
            const int rel = (int)qi - m * BN - 4 * hh;
            const bool diag = m == last;
            if (diag) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int it = 0; it < 16; ++it) {
                        const int off = kb * 32 + 8 * (it >> 2) + (it & 3);
                        if (off > rel) st[kb][it] = -INFINITY;
                    }
            }
            if (WIN && (uint32_t)m * BN + a.window <= q0 + MQ - 1) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int it = 0; it < 16; ++it) {
                        const int off = kb * 32 + 8 * (it >> 2) + (it & 3);
                        if (off <= rel - (int)a.window) st[kb][it] = -INFINITY;   // key before the window
                    }
            }
            bf16x8 dsf[4], dsl[4];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                f32x8 v8;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int kb = cc >> 1, it = (cc & 1) * 8 + j;
                    const float p = fast_exp2(__builtin_fmaf(st[kb][it], a.c, -lse2));
                    if constexpr (SECOND) v8[j] = p * (dpt[kb][it] - dl);   // dS^T
                    else dsum[j & 3] = __builtin_fmaf(p, dpt[kb][it], dsum[j & 3]);
                }
                if constexpr (SECOND) split_bf16(v8, dsf[cc], dsl[cc]);
            }
            if constexpr (SECOND) {
                // dQ^T += K^T dS^T
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) {
                        const bf16x8 kt8 = lds_tr(kt + cc * 16 * ROWB + toff[0][db],
                                                  kt + cc * 16 * ROWB + toff[1][db]);
                        dqt[db] = mfma(kt8, dsf[cc], dqt[db]);
                        dqt[db] = mfma(kt8, dsl[cc], dqt[db]);
                    }
            }
        }
        if constexpr (!SECOND) dl = halves_sum((dsum[0] + dsum[1]) + (dsum[2] + dsum[3]));
        // every wave is done with the ring before the next pass refills it
        __syncthreads();
    };
    pass(std::false_type{});
    if (hh == 0 && qi < a.len) a.delta[srow] = dl;        // for the dK / dV kernel
    pass(std::true_type{});
    // dQ = scale * dQ^T: lane holds dims 32db + 8g + 4hh .. +3 of its row
    if (qi < a.len) {
        uint16_t* orow = a.dq + b * a.q_batch + grp * a.q_group + (uint64_t)h * D + (uint64_t)qi * a.q_row;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 w = {pack_bf16x2(dqt[db][4 * g + 0] * a.scale, dqt[db][4 * g + 1] * a.scale),
                                 pack_bf16x2(dqt[db][4 * g + 2] * a.scale, dqt[db][4 * g + 3] * a.scale)};
                *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * hh) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D, bool WIN>
__global__ void __launch_bounds__(NWK * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
dkv_kernel(const BwdArgs a) {
    constexpr int ROWB = D * 2;
    constexpr int TILE_B = BN * ROWB;
    constexpr int THREADS = NWK * kWave;
    constexpr int LOADS = TILE_B / (THREADS * 16);
    constexpr int DSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int STAGE_B = 2 * TILE_B + 2 * BN * 4;      // Q, dO, lse2, delta
    static_assert(TILE_B % (THREADS * 16) == 0, "tile/thread mismatch");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE_B];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    // work item: (key tile of 128, batch, view, KV head), key tiles ascending
    // (the longest causal extents first)
    const uint32_t per_tile = a.B * a.groups * a.Hkv;
    uint32_t id = blockIdx.x;
    const uint32_t ktile = id / per_tile;
    id %= per_tile;
    const uint32_t kvh = id % a.Hkv;
    id /= a.Hkv;
    const uint32_t grp = id % a.groups;
    const uint32_t b = id / a.groups;
    const uint32_t k0 = ktile * KV_TILE;
    const uint32_t kw0 = k0 + (uint32_t)wave * MQ;       // this wave's first key
    const uint32_t key = kw0 + l32;                      // this lane's key
    const uint32_t kr = min(key, a.len - 1u);

    // K and V fragments (B operands): lane (l32, hh) holds key row, dims 16e + 8hh .. +7
    const uint64_t koff = b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D + (uint64_t)kr * a.kv_row;
    bf16x8 kf[DSTEPS], vf[DSTEPS];
#pragma unroll
    for (int e = 0; e < DSTEPS; ++e) {
        kf[e] = *reinterpret_cast<const bf16x8*>(a.k + koff + (2 * e + hh) * 8);
        vf[e] = *reinterpret_cast<const bf16x8*>(a.v + koff + (2 * e + hh) * 8);
    }

    // stages: (query head of the group, query tile at or after the keys and,
    // with a window, at or before the last query whose window reaches them)
    const uint32_t qt_lo = k0 / BN;
    uint32_t nq = (a.len + BN - 1) / BN;
    if constexpr (WIN) {
        const uint32_t k_last = min(a.len, k0 + KV_TILE) - 1u;
        nq = min(nq, (k_last + a.window - 1u) / BN + 1u);
    }
    const uint32_t per_head = nq - qt_lo;
    const uint32_t n_stage = a.G * per_head;
    const uint32_t q_row_b = (uint32_t)a.q_row * 2u;
    float lse_next = 0.f;                                // wave 0: the next stage's lse, one row per lane
    auto issue = [&](uint32_t t, unsigned char* buf) {
        const uint32_t h = kvh * a.G + t / per_head;
        const uint32_t r0 = (qt_lo + t % per_head) * BN;
        const uint64_t hoff = b * a.q_batch + grp * a.q_group + (uint64_t)h * D;
        const char* qb = reinterpret_cast<const char*>(a.q + hoff) + (uint64_t)r0 * q_row_b;
        const char* ob = reinterpret_cast<const char*>(a.dout + hoff) + (uint64_t)r0 * q_row_b;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const uint32_t lin = (uint32_t)(wave * LOADS + j) * 1024u + (uint32_t)lane * 16u;
            const uint32_t row = lin / ROWB, pch = (lin % ROWB) / 16u;
            const uint32_t sr = min(row, a.len - 1u - r0);
            const uint32_t go = sr * q_row_b + ((pch ^ swz<D>(row)) << 4);
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(qb + go),
                (void __attribute__((address_space(3)))*)(buf + (wave * LOADS + j) * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(ob + go),
                (void __attribute__((address_space(3)))*)(buf + TILE_B + (wave * LOADS + j) * 1024), 16, 0, 0);
        }
        if (wave == 0) {
            // lse and delta of the tile's 64 rows (positions row * groups + grp):
            // delta straight to LDS, lse to a register, which the stage's top
            // scales to log2 units once per row and writes to LDS
            const uint32_t row = min(r0 + (uint32_t)lane, a.len - 1u);
            const uint64_t s = ((uint64_t)b * a.Hq + h) * a.N + (uint64_t)row * a.groups + grp;
            lse_next = a.lse[s];
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(a.delta + s),
                (void __attribute__((address_space(3)))*)(buf + 2 * TILE_B + BN * 4), 4, 0, 0);
        }
    };

    // per-lane LDS offsets (direct reads of Q / dO rows, transpose reads)
    const uint32_t dsw = swz<D>((uint32_t)l32);
    uint32_t doff[DSTEPS];
#pragma unroll
    for (int e = 0; e < DSTEPS; ++e) doff[e] = (uint32_t)l32 * ROWB + ((((uint32_t)(2 * e + hh)) ^ dsw) << 4);
    const uint32_t vg = (uint32_t)lane >> 4, vr = (uint32_t)lane & 15u;
    const uint32_t vk = vr >> 2, va = vr & 3u;
    uint32_t toff[2][DBLK];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const uint32_t row = 4u * (vg >> 1) + vk + 8u * rd;
        const uint32_t sw = swz<D>(row);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const uint32_t lch = 4u * db + 2u * (vg & 1u) + (va >> 1);
            toff[rd][db] = row * ROWB + ((lch ^ sw) << 4) + (va & 1u) * 8u;
        }
    }

    f32x16 dkt[DBLK], dvt[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) {
        dkt[i] = f32x16{};
        dvt[i] = f32x16{};
    }

    if (n_stage > 0) issue(0, smem);
    for (uint32_t t = 0; t < n_stage; ++t) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (wave == 0)
            reinterpret_cast<float*>(smem + (t & 1) * STAGE_B + 2 * TILE_B)[lane] = lse_next * kLog2e;
        __syncthreads();
        if (t + 1 < n_stage) issue(t + 1, smem + ((t + 1) & 1) * STAGE_B);
        const unsigned char* st = smem + (t & 1) * STAGE_B;
        const unsigned char* qt = st;
        const unsigned char* ot = st + TILE_B;
        const float* lt = reinterpret_cast<const float*>(st + 2 * TILE_B);
        const float* dt = lt + BN;
        const uint32_t r0 = (qt_lo + t % per_head) * BN;
#pragma unroll
        for (int qb = 0; qb < BN / MQ; ++qb) {
            const uint32_t rs = r0 + qb * MQ;             // first query of the block
            if (rs + MQ - 1 < kw0 || rs >= a.len) continue;   // all queries before the keys
            if (WIN && rs >= kw0 + MQ - 1 + a.window) continue;   // all past the keys' windows
            // S = Q K^T and dP = dO V^T (32 queries x 32 keys); every fragment
            // read is issued before the products that use it
            bf16x8 qa[DSTEPS], oa[DSTEPS];
#pragma unroll
            for (int e = 0; e < DSTEPS; ++e) {
                qa[e] = lds16(qt + qb * MQ * ROWB + doff[e]);
                oa[e] = lds16(ot + qb * MQ * ROWB + doff[e]);
            }
            // the score products in one block: the wave's K / V fragments stay in
            // the accumulation registers (they are read only here), which leaves
            // the vector registers to S and dP (no moves out of accumulation
            // registers before the softmax).  Entry pad: VALU -> MFMA operand
            // reads; exit pad: MFMA -> VALU result reads.
            f32x16 s, dp;
            if constexpr (DSTEPS == 8) {
                asm volatile("s_nop 4\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q0], %[k0], 0\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o0], %[v0], 0\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q1], %[k1], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o1], %[v1], %[d]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q2], %[k2], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o2], %[v2], %[d]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q3], %[k3], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o3], %[v3], %[d]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q4], %[k4], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o4], %[v4], %[d]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q5], %[k5], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o5], %[v5], %[d]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q6], %[k6], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o6], %[v6], %[d]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q7], %[k7], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o7], %[v7], %[d]\n\t"
                         "s_nop 7\n\t"
                         "s_nop 7\n\t"
                         "s_nop 7\n\t"
                         : [s] "=&v"(s), [d] "=&v"(dp)
                         : [q0] "v"(qa[0]), [q1] "v"(qa[1]), [q2] "v"(qa[2]), [q3] "v"(qa[3]), [q4] "v"(qa[4]), [q5] "v"(qa[5]), [q6] "v"(qa[6]), [q7] "v"(qa[7]), [o0] "v"(oa[0]), [o1] "v"(oa[1]), [o2] "v"(oa[2]), [o3] "v"(oa[3]), [o4] "v"(oa[4]), [o5] "v"(oa[5]), [o6] "v"(oa[6]), [o7] "v"(oa[7]), [k0] "a"(kf[0]), [k1] "a"(kf[1]), [k2] "a"(kf[2]), [k3] "a"(kf[3]), [k4] "a"(kf[4]), [k5] "a"(kf[5]), [k6] "a"(kf[6]), [k7] "a"(kf[7]), [v0] "a"(vf[0]), [v1] "a"(vf[1]), [v2] "a"(vf[2]), [v3] "a"(vf[3]), [v4] "a"(vf[4]), [v5] "a"(vf[5]), [v6] "a"(vf[6]), [v7] "a"(vf[7]));
            } else {
                asm volatile("s_nop 4\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q0], %[k0], 0\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o0], %[v0], 0\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q1], %[k1], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o1], %[v1], %[d]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q2], %[k2], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o2], %[v2], %[d]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[s], %[q3], %[k3], %[s]\n\t"
                         "v_mfma_f32_32x32x16_bf16 %[d], %[o3], %[v3], %[d]\n\t"
                         "s_nop 7\n\t"
                         "s_nop 7\n\t"
                         "s_nop 7\n\t"
                         : [s] "=&v"(s), [d] "=&v"(dp)
                         : [q0] "v"(qa[0]), [q1] "v"(qa[1]), [q2] "v"(qa[2]), [q3] "v"(qa[3]), [o0] "v"(oa[0]), [o1] "v"(oa[1]), [o2] "v"(oa[2]), [o3] "v"(oa[3]), [k0] "a"(kf[0]), [k1] "a"(kf[1]), [k2] "a"(kf[2]), [k3] "a"(kf[3]), [v0] "a"(vf[0]), [v1] "a"(vf[1]), [v2] "a"(vf[2]), [v3] "a"(vf[3]));
            }
            // the transposed operands of dV^T and dK^T, read while P and dS form
            bf16x8 ot8[DBLK][2], qt8[DBLK][2];
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const uint32_t ro = (uint32_t)(qb * MQ + cc * 16) * ROWB;
                    ot8[db][cc] = lds_tr(ot + ro + toff[0][db], ot + ro + toff[1][db]);
                    qt8[db][cc] = lds_tr(qt + ro + toff[0][db], qt + ro + toff[1][db]);
                }
            // lane: key column; entries: query rows 8*(i/4) + 4hh + i%4 of the block
            const int rel = (int)rs + 4 * hh - (int)key;   // query - key = rel + off
            bf16x8 pf[2], pl[2], dsf[2], dsl[2];
            // masks only in blocks that meet the keys' diagonal, the view end or
            // (WIN) the far edge of the keys' windows: a wave-uniform choice, and
            // a select (no branch) per element where they apply
            auto probs = [&](auto masked) __attribute__((always_inline)) {
                constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    f32x8 pv, dv8;
#pragma unroll
                    for (int g2 = 0; g2 < 2; ++g2) {
                        const int g4 = 2 * cc + g2;
                        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + qb * MQ + 8 * g4 + 4 * hh);
                        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + qb * MQ + 8 * g4 + 4 * hh);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int it = 4 * g4 + j;
                            const int off = 8 * g4 + j;
                            float p = fast_exp2(__builtin_fmaf(s[it], a.c, -l4[j]));
                            if constexpr (MASKED) {
                                bool drop = (off + rel < 0) | (rs + (uint32_t)off + 4u * hh >= a.len);
                                if constexpr (WIN) drop = drop | (off + rel >= (int)a.window);
                                p = drop ? 0.f : p;
                            }
                            pv[4 * g2 + j] = p;
                            dv8[4 * g2 + j] = p * (dp[it] - d4[j]);
                        }
                    }
                    split_bf16(pv, pf[cc], pl[cc]);
                    split_bf16(dv8, dsf[cc], dsl[cc]);
                }
            };
            const bool edge = rs < kw0 + MQ || rs + MQ > a.len || (WIN && rs + MQ - 1 >= kw0 + a.window);
            if (edge) probs(std::true_type{});
            else probs(std::false_type{});
            // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    dvt[db] = mfma(ot8[db][cc], pf[cc], dvt[db]);
                    dvt[db] = mfma(ot8[db][cc], pl[cc], dvt[db]);
                    dkt[db] = mfma(qt8[db][cc], dsf[cc], dkt[db]);
                    dkt[db] = mfma(qt8[db][cc], dsl[cc], dkt[db]);
                }
        }
    }
    // dK = scale * dK^T, dV = dV^T: lane holds dims 32db + 8g + 4hh .. +3 of its key
    if (key < a.len) {
        const uint64_t ko = b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D + (uint64_t)key * a.kv_row;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hh;
                const u32x2 wk = {pack_bf16x2(dkt[db][4 * g + 0] * a.scale, dkt[db][4 * g + 1] * a.scale),
                                  pack_bf16x2(dkt[db][4 * g + 2] * a.scale, dkt[db][4 * g + 3] * a.scale)};
                const u32x2 wv = {pack_bf16x2(dvt[db][4 * g + 0], dvt[db][4 * g + 1]),
                                  pack_bf16x2(dvt[db][4 * g + 2], dvt[db][4 * g + 3])};
                *reinterpret_cast<u32x2*>(a.dk + ko + d) = wk;
                *reinterpret_cast<u32x2*>(a.dv + ko + d) = wv;
            }
    }
}

hd_status launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                     int64_t B, int32_t n, int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                     int32_t mode, void* workspace, size_t ws_bytes, hipStream_t stream,
                     int64_t window = 0) {
    // window: 0 = plain causal, else >= 1 (mixing only; checked by the caller)
    if (B < 0 || L < 0 || n < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return HD_ERR_SHAPE;
    if (!scale_ok(scale)) return HD_ERR_SHAPE;
    if (mode != 0 && mode != 1) return HD_ERR_SHAPE;
    if (D != 64 && D != 128) return HD_ERR_UNSUPPORTED;
    if (B == 0 || L == 0) return HD_OK;
    if (!q || !k || !v || !dout || !lse || !dq || !dk || !dv || !workspace) return HD_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
        !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return HD_ERR_SHAPE;
    const int64_t N = (int64_t)n * L;
    if (N > 0x7fffffffLL) return HD_ERR_UNSUPPORTED;
    const uint64_t need = (uint64_t)B * Hq * N * sizeof(float);
    if (ws_bytes < need) return HD_ERR_WORKSPACE;

    const bool within = mode == 0;
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.lse = lse;
    a.delta = static_cast<float*>(workspace);
    a.dq = dq; a.dk = dk; a.dv = dv;
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
    a.Hq = (uint32_t)Hq;
    a.N = (uint32_t)N;
    a.P = (a.G % 8 == 0) ? 8u : (a.G % 4 == 0) ? 4u : ((a.G % 2 == 0) ? 2u : 1u);
    a.n_hpacks = a.G / a.P;
    const uint32_t BT = MQ * (NWQ / a.P);
    a.n_qtiles = (a.len + BT - 1) / BT;
    const uint64_t qitems = (uint64_t)a.n_qtiles * a.B * a.groups * a.Hkv * a.n_hpacks;
    a.n_ktiles = (a.len + KV_TILE - 1) / KV_TILE;
    const uint64_t kitems = (uint64_t)a.n_ktiles * a.B * a.groups * a.Hkv;
    if (qitems > 0x7fffffffULL || kitems > 0x7fffffffULL) return HD_ERR_UNSUPPORTED;
    a.n_items = (uint32_t)qitems;
    a.n_kitems = (uint32_t)kitems;
    a.c = scale * kLog2e;
    a.scale = scale;
    // a window at least as long as the view masks nothing: the causal kernels
    const bool win = window > 0 && window < (int64_t)a.len;
    a.window = win ? (uint32_t)window : 0u;

    // dq_kernel writes delta, which dkv_kernel reads (same stream, in order)
    const dim3 gq(a.n_items), gk(a.n_kitems), bq(NWQ * kWave), bk(NWK * kWave);
    if (D == 128) {
        if (win) {
            dq_kernel<128, true><<<gq, bq, 0, stream>>>(a);
            dkv_kernel<128, true><<<gk, bk, 0, stream>>>(a);
        } else {
            dq_kernel<128, false><<<gq, bq, 0, stream>>>(a);
            dkv_kernel<128, false><<<gk, bk, 0, stream>>>(a);
        }
    } else {
        if (win) {
            dq_kernel<64, true><<<gq, bq, 0, stream>>>(a);
            dkv_kernel<64, true><<<gk, bk, 0, stream>>>(a);
        } else {
            dq_kernel<64, false><<<gq, bq, 0, stream>>>(a);
            dkv_kernel<64, false><<<gk, bk, 0, stream>>>(a);
        }
    }
    return launch_status();
}

}  // namespace

}  // namespace hdsfa

extern "C" size_t sfa_attn_bwd_workspace_size(int64_t B, int32_t n, int64_t L, int32_t Hq) {
    if (B < 0 || n < 1 || L < 0 || Hq < 1) return 0;
    return (size_t)B * (size_t)Hq * (size_t)n * (size_t)L * sizeof(float);
}

extern "C" hd_status sfa_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const uint16_t* dout, const float* lse,
                                  uint16_t* dq, uint16_t* dk, uint16_t* dv, int64_t B, int32_t n,
                                  int64_t L, int32_t Hq, int32_t Hkv, int32_t D,
                                  float softmax_scale, int32_t mode, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    return hdsfa::launch_bwd(q, k, v, dout, lse, dq, dk, dv, B, n, L, Hq, Hkv, D, softmax_scale,
                             mode, workspace, workspace_bytes, stream);
}

extern "C" hd_status sfa_attn_bwd_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         const uint16_t* dout, const float* lse,
                                         uint16_t* dq, uint16_t* dk, uint16_t* dv, int64_t B,
                                         int32_t n, int64_t L, int32_t Hq, int32_t Hkv, int32_t D,
                                         float softmax_scale, int64_t window, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    if (window < 1 || window > 0x7fffffffLL) return HD_ERR_SHAPE;
    return hdsfa::launch_bwd(q, k, v, dout, lse, dq, dk, dv, B, n, L, Hq, Hkv, D, softmax_scale,
                             /*mode=*/1, workspace, workspace_bytes, stream, window);
}

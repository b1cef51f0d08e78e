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
constexpr int NW = 8;        // waves per workgroup (2 per SIMD)
constexpr int NSTAGE = 3;    // LDS ring depth for K and for V tiles
constexpr int THREADS = NW * kWave;

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
    uint32_t P;          // query heads packed per workgroup (1, 2, 4 or 8)
    uint32_t n_hpacks;   // G / P
    uint32_t n_qtiles;   // ceil(len / (MQ * NW / P))
    float c;             // softmax scale * log2(e)
};

// XOR swizzle of the 16-byte chunks of a K/V row in LDS (rows of D bf16 =
// D/8 chunks).  Two read patterns must hit distinct banks:
//   K:  16 consecutive rows, one logical chunk each (16-byte reads);
//   V:  per 32 lanes, 4 consecutive rows x 4 consecutive logical chunks
//       (8-byte transpose reads).
// D=128 (256-byte rows span all 64 banks): swz = (r%4)*4 + (r/4)%4.
// D=64 (128-byte rows, even/odd rows on opposite bank halves): the same idea
// over rows of one parity: swz = ((r/2)%2)*4 + (r/4)%4.
template <int D>
__device__ __forceinline__ uint32_t swz(uint32_t row) {
    if constexpr (D == 128) return ((row & 3u) << 2) | ((row >> 2) & 3u);
    else return (((row >> 1) & 1u) << 2) | ((row >> 2) & 3u);
}

// Eight transpose reads of V for one 32-dim block: the two key quads (rd = 0,
// 1) of each of the four 16-key steps c (immediate offsets c * 16 rows).  The
// reads are issued from inline assembly so that the compiler does not order
// them behind the asynchronous global->LDS loads of the next tile, which
// target the other LDS stage; the block waits for its own results before it
// returns, so every output register is complete when the asm ends.
template <int ROWB>
__device__ __forceinline__ void v_tr_reads(uint32_t a0, uint32_t a1, u32x2 (&r)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%10\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%11\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]),
          "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a0), "v"(a1), "i"(16 * ROWB), "i"(32 * ROWB), "i"(48 * ROWB)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int D>
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
sfa_prefill_kernel(const PrefillArgs a) {
    constexpr int ROWB = D * 2;                // bytes per K/V row
    constexpr int TILE_B = BN * ROWB;          // one K (or V) tile
    constexpr int STAGE_B = 2 * TILE_B;        // K tile then V tile
    constexpr int LOADS = TILE_B / (THREADS * 16);   // 16-byte direct loads per thread per tile
    constexpr int DSTEPS = D / 16;             // k-steps of the score product
    constexpr int DBLK = D / 32;               // 32-row blocks of O^T
    static_assert(TILE_B % (THREADS * 16) == 0, "tile/thread mismatch");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * STAGE_B];   // K ring, V ring

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
    const char* kview = reinterpret_cast<const char*>(a.k + b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D);
    const char* vview = reinterpret_cast<const char*>(a.v + b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D);

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

    // ---- direct global->LDS tile loads ----
    // Load j of this wave fills LDS bytes [(wave*LOADS + j)*1024, +1024) of a
    // tile, lane i its 16 bytes at +16*i: tile row r, physical chunk p, which
    // holds logical chunk p ^ swz(r).  Rows past the view end (last tile only)
    // are clamped to the last valid row: such keys lie in the future of every
    // valid query, the causal mask gives them probability 0, and the finite
    // values they hold never reach the output.
    const uint32_t kv_row_b = (uint32_t)a.kv_row * 2u;
    uint32_t ld_row[LOADS], ld_off[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const uint32_t lin = (uint32_t)(wave * LOADS + j) * 1024u + (uint32_t)lane * 16u;
        const uint32_t row = lin / ROWB;
        const uint32_t pch = (lin % ROWB) / 16u;
        ld_row[j] = row;
        ld_off[j] = row * kv_row_b + ((pch ^ swz<D>(row)) << 4);
    }
    auto issue = [&](const char* view, int kt, unsigned char* buf) {
        const uint32_t k0 = (uint32_t)kt * BN;
        const char* base = view + (uint64_t)k0 * kv_row_b;
        const bool full = k0 + BN <= a.len;
        const uint32_t last = a.len - 1 - k0;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            uint32_t off = ld_off[j];
            if (!full) off -= (ld_row[j] - min(ld_row[j], last)) * kv_row_b;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(base + off),
                (void __attribute__((address_space(3)))*)(buf + (wave * LOADS + j) * 1024), 16, 0, 0);
        }
    };

    // ---- per-lane LDS read offsets (independent of the tile) ----
    // K (A operand of S^T = K Q^T): row kb*32 + l32, logical chunk 2e + hh.
    const uint32_t kswz = swz<D>((uint32_t)l32);
    uint32_t koff[DSTEPS];
#pragma unroll
    for (int e = 0; e < DSTEPS; ++e)
        koff[e] = (uint32_t)l32 * ROWB + ((((uint32_t)(2 * e + hh)) ^ kswz) << 4);
    // V (A operand of O^T = V^T P^T) through the transpose read: in each
    // 16-lane group g, lane r = 4k + a addresses key row (16c + 4*(g/2) + k +
    // 8*rd) at dims 32db + 16*(g%2) + 4a; lane i of the group then receives
    // dim 32db + 16*(g%2) + i of those 4 keys, i.e. 4 of the 8 keys that the
    // P^T operand holds in the same slots.
    const uint32_t vg = (uint32_t)lane >> 4, vr = (uint32_t)lane & 15u;
    const uint32_t vk = vr >> 2, va = vr & 3u;
    uint32_t voff[2][DBLK];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
        const uint32_t key = 4u * (vg >> 1) + vk + 8u * rd;
        const uint32_t sw = swz<D>(key);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const uint32_t lch = 4u * db + 2u * (vg & 1u) + (va >> 1);
            voff[rd][db] = key * ROWB + ((lch ^ sw) << 4) + (va & 1u) * 8u;
        }
    }

    // S^T[key][query] = K Q^T for the two 32-key blocks of a tile
    auto qk = [&](const unsigned char* ks, f32x16 (&sacc)[BN / 32]) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) sacc[kb] = f32x16{};
#pragma unroll
        for (int e = 0; e < DSTEPS; ++e)
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + kb * 32 * ROWB + koff[e]);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[e], sacc[kb], 0, 0, 0);
            }
    };

    // online softmax of one tile's scores; returns the P^T operands.  The
    // causal mask is needed only on a wave's last (diagonal) tile.
    auto softmax = [&](f32x16 (&sacc)[BN / 32], int kt, bool diag, bf16x8 (&pf)[BN / 16]) {
        if (diag) {
            const uint32_t k0 = (uint32_t)kt * BN;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int it = 0; it < 16; ++it) {
                    const uint32_t key = k0 + kb * 32 + 8 * (it >> 2) + 4 * hh + (it & 3);
                    if (key > qi) sacc[kb][it] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int it = 0; it < 16; ++it) mx = fmaxf(mx, sacc[kb][it]);
        mx = halves_max(mx) * a.c;
        // Lazy rescale: the reference max m_run only moves when a row's tile
        // max exceeds it by more than 8 (a factor 2^8), so O and l are
        // rescaled rarely (always on the first tile).  Probabilities stay
        // <= 2^8 and the result O / l is unchanged.
        if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.f) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < DBLK; ++i) oacc[i] *= alpha;
        }
        float rsp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const float p = fast_exp2(__builtin_fmaf(sacc[kb][it], a.c, -m_run));
                sacc[kb][it] = p;
                rsp[it & 3] += p;
            }
        l_run += halves_sum((rsp[0] + rsp[1]) + (rsp[2] + rsp[3]));
        // P^T fragments (B operand): 16-key step c takes items 8*(c%2)..+7
#pragma unroll
        for (int c = 0; c < BN / 16; ++c) {
            const f32x16& s = sacc[c >> 1];
            const int o8 = (c & 1) * 8;
            pf[c] = to_bf16x8(f32x8{s[o8 + 0], s[o8 + 1], s[o8 + 2], s[o8 + 3],
                                    s[o8 + 4], s[o8 + 5], s[o8 + 6], s[o8 + 7]});
        }
    };

    // O^T[d][query] += V^T P^T
    auto pv = [&](const unsigned char* vs, const bf16x8 (&pf)[BN / 16]) {
        static_assert(BN == 64, "the transpose-read helper covers 4 steps of 16 keys");
        const uint32_t vbase = lds_addr(vs);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            u32x2 vr8[8];
            v_tr_reads<ROWB>(vbase + voff[0][db], vbase + voff[1][db], vr8);
#pragma unroll
            for (int c = 0; c < BN / 16; ++c) {
                const u32x4 w = {vr8[2 * c][0], vr8[2 * c][1], vr8[2 * c + 1][0], vr8[2 * c + 1][1]};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, w), pf[c], oacc[db], 0, 0, 0);
            }
        }
    };

    // ---- software pipeline over key tiles ----
    // LDS holds a ring of NSTAGE K tiles and one of NSTAGE V tiles.  Step j
    // computes S(j+1) = K(j+1) Q^T while it turns S(j) into probabilities and
    // accumulates P(j) V(j).  K(t) is last read in step t-1 and V(t) in step
    // t, so at the top of step j (after the barrier) the slots of K(j) and
    // V(j-1) are free and receive K(j+3) and V(j+2): every tile is requested
    // two steps before it is used.
    auto kbuf = [&](int t) { return smem + (t % NSTAGE) * TILE_B; };
    auto vbuf = [&](int t) { return smem + (NSTAGE + t % NSTAGE) * TILE_B; };

    issue(kview, 0, kbuf(0));
    issue(vview, 0, vbuf(0));
    if (n_kt > 1) { issue(kview, 1, kbuf(1)); issue(vview, 1, vbuf(1)); }
    if (n_kt > 2) issue(kview, 2, kbuf(2));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 sa[BN / 32], sb[BN / 32];
    if (wave_kt > 0) qk(kbuf(0), sa);

    // one pipeline step; the loop below alternates the two score buffers so
    // that S(j+1) never has to be copied into S(j)'s registers
    int in_flight = 0;      // direct loads this thread issued in the previous step
    auto step = [&](int j, f32x16 (&s_cur)[BN / 32], f32x16 (&s_next)[BN / 32]) {
        // K(j+1) and V(j) were requested two steps ago: wait until only the
        // previous step's requests may still be in flight, then make every
        // wave's data visible (and every wave done with K(j), V(j-1))
        if (in_flight == 2 * LOADS) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * LOADS) : "memory");
        else if (in_flight == LOADS) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LOADS) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // a bare barrier: the wait above already covers the loads this step
        // needs, and a release fence here would also wait for the requests
        // still in flight for later steps
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        in_flight = 0;
        if (j + 3 < n_kt) { issue(kview, j + 3, kbuf(j + 3)); in_flight += LOADS; }
        if (j + 2 < n_kt) { issue(vview, j + 2, vbuf(j + 2)); in_flight += LOADS; }

        // this wave's last key tile holds its diagonal and needs the mask
        const int last = wave_kt - 1;
        if (j < last) {
            // hot path: S(j+1) = K(j+1) Q^T interleaved with the softmax of S(j)
            bf16x8 pf[BN / 16];
            qk(kbuf(j + 1), s_next);
            softmax(s_cur, j, false, pf);
            // 16 x {one K fragment read, one MFMA, a slice of softmax VALU}
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // VALU
            }
            pv(vbuf(j), pf);
        } else if (j == last) {
            bf16x8 pf[BN / 16];
            softmax(s_cur, j, true, pf);
            pv(vbuf(j), pf);
        }
    };
    for (int j = 0; j < n_kt; j += 2) {
        step(j, sa, sb);
        if (j + 1 < n_kt) step(j + 1, sb, sa);
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
    a.P = (a.G % 8 == 0) ? 8u : (a.G % 4 == 0) ? 4u : ((a.G % 2 == 0) ? 2u : 1u);
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

// Hidden Decoding decode step over the retained per-stream KV cache
// (sfa_decode_workspace_size, sfa_decode_step, sfa_decode_step_window,
// sfa_decode_step_paged, and sfa_decode_step_noalloc, which keeps the split
// partials in a static per-device array instead of a caller's workspace).
//
// "Hidden Decoding at Scale" review, sections Method and Limitations: the KV
// of every stream is kept, so the cache holds n entries per token and later
// tokens read all of them; section Notes: small-batch decode is bound by
// memory bandwidth.  Each step appends the n new stream positions of the next
// token and attends from them.
//
// Three kernels on the caller's stream:
//   1. append   -- copies k_new/v_new into entries T*n .. T*n+n-1;
//   2. attend   -- split-K over a strided view of the cache.  Within-stream
//                  mode: one view per stream s (entries s, s+n, ..., T*n+s),
//                  whose G query rows all sit at its last entry, so no mask
//                  is needed.  Mixing mode: one view of all (T+1)*n entries
//                  with n*G query rows, causal only among the n new entries.
//                  Either way every cache byte is read exactly once per call.
//                  K and V tiles are staged through LDS row-major with
//                  coalesced loads (16 lanes per 256-byte row; the V^T
//                  operand comes from transpose reads) and both contractions
//                  run on v_mfma_f32_32x32x16_bf16; 4 waves take 32 keys each
//                  of a 128-key tile and merge their (max, sum, O) at the end;
//   3. combine  -- merges the per-split partials (fp32) into bf16 output
//                  (skipped when every view is one split: the attention
//                  kernel then writes the normalised bf16 rows itself).
// Sliding-window mixing (sfa_decode_step_window; the review's Method: mixing
// layers follow the base model's pattern, sliding-window or full): query
// (T, s) at p = T*n + s reads entries p - W < j <= p, so the view starts at
// T*n - W + 1 and only W + n - 1 entries per sequence are read.
// Paged caches (sfa_decode_step_paged): entry e of sequence q lives in page
// page_table[q, e / P], slot e % P (P a power of two) of a pool of pages; the
// same kernels look every cache row up through the table (PAGED instances).
// No atomics: results are bitwise reproducible run to run.
#include "common.h"

#include <mutex>

namespace hdsfa {

namespace {

constexpr int DT = 128;            // keys per workgroup tile (32 per wave)
constexpr int DNW = 4;             // waves
constexpr int DTHREADS = DNW * kWave;
constexpr int kTargetBlocks = 512;    // split-plan target: two resident workgroups on each of 256 CUs

typedef short v4i16 __attribute__((ext_vector_type(4)));
// an LDS address for the transpose read (the pointer points into __shared__ memory)
__device__ __forceinline__ __attribute__((address_space(3))) v4i16* lds_v4(const uint16_t* p) {
    return (__attribute__((address_space(3))) v4i16*)(p);
}

struct DecodeArgs {
    const uint16_t* q;         // [S, n, Hq, D]
    const uint16_t* kc;        // [S, C, Hkv, D]
    const uint16_t* vc;
    const int32_t* tokens_before;
    float* ws;
    uint64_t cache_seq;        // C * Hkv * D
    uint32_t n, Hq, Hkv, G, R; // R = n*G query rows per KV head
    uint32_t max_tokens;
    uint32_t nsplit, split;    // splits per view, keys per split (multiple of DT)
    uint32_t within;
    uint32_t window;           // mixing only: 0 = full pattern, else W
    float c;
    const int32_t* page_table; // [S, mpps] (PAGED instances)
    uint32_t pshift, mpps, num_pages;
    uint16_t* out;             // [S, n, Hq, D]: written here when direct
    uint32_t direct;           // one split per view: the merged row is the output
    int32_t* err;              // NULL or the caller's flag: set to 1 on an out-of-range page id
};

// true when a page id lies outside the pool (it is then clamped into it)
__device__ __forceinline__ bool page_out_of_range(int32_t pg, uint32_t num_pages) {
    return pg < 0 || pg >= (int32_t)num_pages;
}

// pool row of entry e of sequence seq (page ids outside the pool are clamped
// into it, so no access leaves the pool; `bad` is set for such an id)
__device__ __forceinline__ uint64_t paged_row(const int32_t* __restrict__ pt, uint32_t seq, uint32_t e,
                                              uint32_t pshift, uint32_t mpps, uint32_t num_pages,
                                              bool& bad) {
    const uint32_t slot = min(e >> pshift, mpps - 1u);
    int32_t pg = pt[(uint64_t)seq * mpps + slot];
    bad = bad || page_out_of_range(pg, num_pages);
    pg = pg < 0 ? 0 : (pg >= (int32_t)num_pages ? (int32_t)num_pages - 1 : pg);
    return ((uint64_t)(uint32_t)pg << pshift) | (e & ((1u << pshift) - 1u));
}

// first entry of a view that any of the n new queries can see
__device__ __forceinline__ uint32_t view_start(uint32_t T, uint32_t n, uint32_t window) {
    const uint32_t p0 = T * n;
    return (window != 0u && p0 + 1u >= window) ? p0 + 1u - window : 0u;
}

__device__ __forceinline__ uint32_t clamp_tokens(int32_t t, uint32_t max_tokens) {
    return t < 0 ? 0u : ((uint32_t)t > max_tokens ? max_tokens : (uint32_t)t);
}

// ---------------------------------------------------------------------------
// 1. append
// ---------------------------------------------------------------------------
template <bool PAGED>
__global__ void __launch_bounds__(256)
decode_append_kernel(const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
                     u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                     const int32_t* __restrict__ tokens_before, uint32_t S, uint32_t n,
                     uint32_t row_chunks /* Hkv*D/8 */, uint64_t cache_seq_chunks,
                     uint32_t max_tokens, const int32_t* __restrict__ pt, uint32_t pshift,
                     uint32_t mpps, uint32_t num_pages, int32_t* __restrict__ err) {
    const uint32_t idx = blockIdx.x * 256 + threadIdx.x;
    const uint32_t per_seq = n * row_chunks;
    if (idx >= S * per_seq) return;
    const uint32_t seq = idx / per_seq;
    const uint32_t rem = idx - seq * per_seq;      // s*row_chunks + w
    const int32_t raw = tokens_before[seq];
    const uint32_t T = clamp_tokens(raw, max_tokens);
    // every kernel of the step clamps tokens_before the same way; this one,
    // which reads every sequence's count, reports a count outside [0, max_tokens]
    bool bad = raw < 0 || (uint32_t)raw > max_tokens;
    uint64_t dst;
    if constexpr (PAGED) {
        const uint32_t s = rem / row_chunks;
        dst = paged_row(pt, seq, T * n + s, pshift, mpps, num_pages, bad) * row_chunks + (rem - s * row_chunks);
    } else {
        dst = seq * cache_seq_chunks + (uint64_t)T * n * row_chunks + rem;
    }
    if (bad && err != nullptr) *err = 1;
    kc[dst] = k_new[idx];
    vc[dst] = v_new[idx];
}

// ---------------------------------------------------------------------------
// 2. split-K attention
// ---------------------------------------------------------------------------
// One register set of tiles in flight.  With NQB = 1 two workgroups fit on a
// compute unit, and each covers the other's load waits, start and merge (a
// second register set would need the whole register file: one workgroup per
// unit, measured slower; with NQB = 2 it spilled).
template <int D, int NQB, bool PAGED>
__global__ void __launch_bounds__(DTHREADS) __attribute__((amdgpu_waves_per_eu(NQB == 1 ? 2 : 1, 2)))
decode_attend_kernel(const DecodeArgs a) {
    constexpr int KP = D + 8;
    constexpr int KS_ELEMS = DT * KP;
    constexpr int DSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int CPR = D / 8;
    constexpr int K_CHUNKS = DT * CPR / DTHREADS;
    static_assert((DT * CPR) % DTHREADS == 0, "tile/thread mismatch");
    // V rows are padded to D + 32 elements: the 4 rows a 16-lane group reads
    // in one transpose read then start 16 banks apart
    constexpr int VP = D + 32;
    // LDS: K tile + V tile (both row-major); reused for the cross-wave merge
    constexpr int TILE_ELEMS = KS_ELEMS + DT * VP;
    constexpr int MERGE_FLOATS = DNW * NQB * 32 * D;
    constexpr int SMEM_BYTES = (TILE_ELEMS * 2 > MERGE_FLOATS * 4) ? TILE_ELEMS * 2 : MERGE_FLOATS * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SMEM_BYTES];
    __shared__ float sm_m[DNW][NQB * 32];
    __shared__ float sm_l[DNW][NQB * 32];
    // PAGED: pool row of each key of the next two tiles (slot = tile parity)
    __shared__ uint32_t row_tab[PAGED ? 2 * DT : 1];
    uint16_t* ks = reinterpret_cast<uint16_t*>(smem_raw);
    uint16_t* vs = ks + KS_ELEMS;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const uint32_t sp = blockIdx.x;
    const uint32_t views = a.within ? a.n : 1u;
    const uint32_t view = blockIdx.y % views;
    const uint32_t kvh = blockIdx.y / views;
    const uint32_t seq = blockIdx.z;

    const uint32_t T = clamp_tokens(a.tokens_before[seq], a.max_tokens);
    const uint32_t len = a.within ? T + 1 : (T + 1) * a.n;     // keys in the view
    const uint32_t lo = a.within ? 0u : view_start(T, a.n, a.window);
    const uint32_t key0 = lo + sp * a.split;
    if (key0 >= len) return;                                    // whole block idle
    const uint32_t key_end = min(len, key0 + a.split);
    const int n_tiles = (int)((key_end - key0 + DT - 1) / DT);

    // view rows: key index i of the view is cache entry i*rstride + view
    const uint32_t rstride = a.within ? a.n : 1u;
    const uint64_t erow = (uint64_t)a.Hkv * D;                  // elements per cache entry
    const uint16_t* kbase = a.kc + seq * a.cache_seq + (uint64_t)view * erow + (uint64_t)kvh * D;
    const uint16_t* vbase = a.vc + seq * a.cache_seq + (uint64_t)view * erow + (uint64_t)kvh * D;
    const uint64_t kstep = (uint64_t)rstride * erow;

    // query rows of this view: within -> the G heads of stream `view`;
    // mixing -> r = s*G + gh for every stream s.
    const uint32_t rows = a.within ? a.G : a.R;
    bf16x8 qf[NQB][DSTEPS];
    uint32_t qidx[NQB];                                          // last visible key
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const uint32_t rl = qb * 32 + l32;
        const bool ok = rl < rows;
        const uint32_t r = a.within ? view * a.G + rl : rl;
        const uint32_t s = r / a.G;
        const uint32_t gh = r - s * a.G;
        qidx[qb] = a.within ? T : T * a.n + s;
        const u32x4* src = reinterpret_cast<const u32x4*>(
            a.q + (((uint64_t)seq * a.n + s) * a.Hq + kvh * a.G + gh) * D);
#pragma unroll
        for (int e = 0; e < DSTEPS; ++e) {
            u32x4 w = ok ? src[2 * e + hh] : u32x4{0u, 0u, 0u, 0u};
            qf[qb][e] = __builtin_bit_cast(bf16x8, w);
        }
    }

    f32x16 oacc[NQB][DBLK];
    float m_run[NQB], l_run[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
#pragma unroll
        for (int i = 0; i < DBLK; ++i) oacc[qb][i] = f32x16{};
    }

    // Tiles go global -> registers -> LDS: the next tile (64 KB per
    // workgroup) is in flight while the current one is consumed from LDS.
    // K and V use the same pattern: 16 consecutive lanes read one key's
    // 256-byte row, so every load instruction covers whole rows (gathering
    // 4 keys per lane for a register transpose of V instead cost 4-10%).
    // Rows past the split end are clamped to its last row: the mask below
    // gives them probability 0.
    // PAGED: the pool rows of a tile's keys come from row_tab, filled two
    // tiles ahead: the load of tile t also fetches (threads < DT, one key
    // each) the page id of tile t+2 into pg, and the LDS store of tile t
    // turns it into a pool row.  The data loads thus never wait on a table
    // lookup (loads return in issue order, so a lookup issued just before
    // them would also drain the tile already in flight).
    struct TileRegs {
        u32x4 k[K_CHUNKS];
        u32x4 v[K_CHUNKS];
        int32_t pg;       // PAGED: raw page id of this thread's key of tile t+2
        uint32_t pg_lo;   //        and that key's slot within its page
    };
    const uint32_t last_key = key_end - 1;
    const uint32_t pmask = (1u << a.pshift) - 1u;
    // page id (raw) and slot of key j of tile t; keys past the split are clamped
    auto fetch_page = [&](int t, int j, int32_t& pg, uint32_t& lo) {
        const uint32_t key = min(key0 + (uint32_t)t * DT + (uint32_t)j, last_key);
        const uint32_t e = key * rstride + view;
        const uint32_t slot = min(e >> a.pshift, a.mpps - 1u);
        pg = a.page_table[(uint64_t)seq * a.mpps + slot];
        lo = e & pmask;
    };
    auto pool_row = [&](int32_t pg, uint32_t lo) -> uint32_t {
        pg = pg < 0 ? 0 : (pg >= (int32_t)a.num_pages ? (int32_t)a.num_pages - 1 : pg);
        return ((uint32_t)pg << a.pshift) | lo;
    };
    auto load_tile = [&](int t, TileRegs& r, int slot) {
        const uint32_t k0 = key0 + (uint32_t)t * DT;
        [[maybe_unused]] const uint32_t* tab = row_tab + slot * DT;
#pragma unroll
        for (int i = 0; i < K_CHUNKS; ++i) {
            const int cidx = tid + i * DTHREADS;
            if constexpr (PAGED) {
                const uint64_t row = tab[cidx / CPR];
                r.k[i] = *reinterpret_cast<const u32x4*>(a.kc + row * erow + (uint64_t)kvh * D + (cidx % CPR) * 8);
            } else {
                const uint32_t key = min(k0 + cidx / CPR, last_key);
                r.k[i] = *reinterpret_cast<const u32x4*>(kbase + key * kstep + (cidx % CPR) * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < K_CHUNKS; ++i) {
            const int cidx = tid + i * DTHREADS;
            if constexpr (PAGED) {
                const uint64_t row = tab[cidx / CPR];
                r.v[i] = *reinterpret_cast<const u32x4*>(a.vc + row * erow + (uint64_t)kvh * D + (cidx % CPR) * 8);
            } else {
                const uint32_t key = min(k0 + cidx / CPR, last_key);
                r.v[i] = *reinterpret_cast<const u32x4*>(vbase + key * kstep + (cidx % CPR) * 8);
            }
        }
        if constexpr (PAGED) {
            if (tid < DT) fetch_page(t + 2, tid, r.pg, r.pg_lo);
        }
    };
    auto store_tile = [&](const TileRegs& r, int slot) {
        if constexpr (PAGED) {
            if (tid < DT) {
                if (page_out_of_range(r.pg, a.num_pages) && a.err != nullptr) *a.err = 1;
                row_tab[slot * DT + tid] = pool_row(r.pg, r.pg_lo);
            }
        }
#pragma unroll
        for (int i = 0; i < K_CHUNKS; ++i) {
            const int cidx = tid + i * DTHREADS;
            const int row = cidx / CPR;
            const int col = cidx % CPR;
            *reinterpret_cast<u32x4*>(ks + row * KP + col * 8) = r.k[i];
        }
#pragma unroll
        for (int i = 0; i < K_CHUNKS; ++i) {
            const int cidx = tid + i * DTHREADS;
            const int row = cidx / CPR;
            const int col = cidx % CPR;
            *reinterpret_cast<u32x4*>(vs + row * VP + col * 8) = r.v[i];
        }
    };

    // V^T operand of O^T += V^T P^T from the row-major V tile by transpose
    // reads (ds_read_b64_tr_b16): the 16 lanes of group g = lane / 16 each
    // address 4 dims (4 * (lane % 4)) of one of 4 key rows (lane % 16 / 4);
    // lane i of the group receives dim 16 * (g % 2) + i of those 4 keys.
    // Groups 0-1 take keys 0-3, groups 2-3 keys 4-7 of each 8-key half; the
    // second read (+8 keys) completes the 8 k-slots, which then hold keys
    // 4*hh + {0..3, 8..11} in the order the P^T operand holds them.
    const uint16_t* vlane = vs + (wave * 32 + 4 * (lane >> 5) + ((lane & 15) >> 2)) * VP +
                            16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto compute = [&](int t) {
        const uint32_t wk0 = key0 + (uint32_t)t * DT + wave * 32;   // this wave's first key
        if (wk0 >= key_end) return;
        f32x16 sacc[NQB];
        const uint16_t* krow = ks + (wave * 32 + l32) * KP + hh * 8;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) sacc[qb] = f32x16{};
#pragma unroll
        for (int e = 0; e < DSTEPS; ++e) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 16 * e);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
                sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][e], sacc[qb], 0, 0, 0);
        }

        bf16x8 pf[NQB][2];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            // keys past the view end, after the query (mixing, new token) or
            // before its window -> -inf
            const bool below = a.window != 0u && wk0 + a.window <= qidx[qb];
            if (wk0 + 31 > qidx[qb] || wk0 + 31 >= key_end || below) {
#pragma unroll
                for (int it = 0; it < 16; ++it) {
                    const uint32_t key = wk0 + 8 * (it >> 2) + 4 * hh + (it & 3);
                    if (key > qidx[qb] || key >= key_end || (a.window != 0u && key + a.window <= qidx[qb]))
                        sacc[qb][it] = -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int it = 0; it < 16; ++it) mx = fmaxf(mx, sacc[qb][it]);
            mx = halves_max(mx);
            const float m_new = fmaxf(m_run[qb], mx * a.c);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[qb] - m_use);
            m_run[qb] = m_new;
            float rsp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const float p = fast_exp2(__builtin_fmaf(sacc[qb][it], a.c, -m_use));
                sacc[qb][it] = p;
                rsp[it & 3] += p;
            }
            l_run[qb] = l_run[qb] * alpha + halves_sum((rsp[0] + rsp[1]) + (rsp[2] + rsp[3]));
#pragma unroll
            for (int i = 0; i < DBLK; ++i) oacc[qb][i] *= alpha;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int o8 = c * 8;
                pf[qb][c] = to_bf16x8(f32x8{sacc[qb][o8 + 0], sacc[qb][o8 + 1], sacc[qb][o8 + 2],
                                            sacc[qb][o8 + 3], sacc[qb][o8 + 4], sacc[qb][o8 + 5],
                                            sacc[qb][o8 + 6], sacc[qb][o8 + 7]});
            }
        }
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint16_t* src = vlane + (16 * c) * VP + 32 * db;
                const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4(src));
                const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_v4(src + 8 * VP));
                const u32x2 lo = __builtin_bit_cast(u32x2, lo4), hi = __builtin_bit_cast(u32x2, hi4);
                const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][c], oacc[qb][db], 0, 0, 0);
            }
        }
    };

    // tile t reads row_tab slot t & 1; the store of tile t fills that slot
    // with tile t+2's rows once every load of tile t has read it (a barrier
    // lies between them: the one after the previous compute, or for tile 0
    // the one after its load)
    if constexpr (PAGED) {
        if (tid < DT) {
            int32_t pg0, pg1;
            uint32_t lo0, lo1;
            fetch_page(0, tid, pg0, lo0);
            fetch_page(1, tid, pg1, lo1);
            if ((page_out_of_range(pg0, a.num_pages) || page_out_of_range(pg1, a.num_pages)) &&
                a.err != nullptr)
                *a.err = 1;
            row_tab[tid] = pool_row(pg0, lo0);
            row_tab[DT + tid] = pool_row(pg1, lo1);
        }
        __syncthreads();
    }
    TileRegs r;
    load_tile(0, r, 0);
    if constexpr (PAGED) __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        store_tile(r, t & 1);
        __syncthreads();
        if (t + 1 < n_tiles) load_tile(t + 1, r, (t + 1) & 1);
        compute(t);
        __syncthreads();
    }

    // ---- merge the 4 waves' partial softmax states through LDS ----
    float* mo = reinterpret_cast<float*>(smem_raw);          // [wave][row][d]
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int row = qb * 32 + l32;
        if (hh == 0) {
            sm_m[wave][row] = m_run[qb];
            sm_l[wave][row] = l_run[qb];
        }
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int d = db * 32 + 8 * (it >> 2) + 4 * hh + (it & 3);
                mo[(wave * NQB * 32 + row) * D + d] = oacc[qb][db][it];
            }
    }
    __syncthreads();

    const uint32_t r_base = a.within ? view * a.G : 0u;
    for (int idx = tid; idx < (int)rows * D; idx += DTHREADS) {
        const int row = idx / D;
        const int d = idx - row * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < DNW; ++w) M = fmaxf(M, sm_m[w][row]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < DNW; ++w) {
            const float f = fast_exp2(sm_m[w][row] - Mu);
            o += f * mo[(w * NQB * 32 + row) * D + d];
            l += f * sm_l[w][row];
        }
        const uint32_t r = r_base + row;
        if (a.direct) {
            // the combine of a single split: its weight is 2^0 = 1, so the
            // output is o / l rounded to bf16
            const uint32_t s = r / a.G;
            const uint32_t gh = r - s * a.G;
            const __bf16 hv = (__bf16)(o / l);
            a.out[(((uint64_t)seq * a.n + s) * a.Hq + kvh * a.G + gh) * D + d] = __builtin_bit_cast(uint16_t, hv);
            continue;
        }
        float* part = a.ws + ((((uint64_t)seq * a.Hkv + kvh) * a.R + r) * a.nsplit + sp) * (D + 2);
        if (d == 0) {
            part[0] = M;
            part[1] = l;
        }
        part[2 + d] = o;
    }
}

// ---------------------------------------------------------------------------
// 3. combine
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
decode_combine_kernel(const float* __restrict__ ws, const int32_t* __restrict__ tokens_before,
                      uint16_t* __restrict__ out, uint32_t S, uint32_t n, uint32_t Hq,
                      uint32_t Hkv, uint32_t G, uint32_t R, uint32_t nsplit, uint32_t split,
                      uint32_t within, uint32_t max_tokens, uint32_t window) {
    const uint32_t idx = blockIdx.x * 256 + threadIdx.x;    // over S*Hkv*R*D
    if (idx >= S * Hkv * R * D) return;
    const uint32_t d = idx % D;
    const uint32_t unit = idx / D;                             // (seq*Hkv + kvh)*R + r
    const uint32_t r = unit % R;
    const uint32_t sk = unit / R;
    const uint32_t kvh = sk % Hkv;
    const uint32_t seq = sk / Hkv;
    const uint32_t T = clamp_tokens(tokens_before[seq], max_tokens);
    const uint32_t len = within ? T + 1 : (T + 1) * n;
    const uint32_t lo = within ? 0u : view_start(T, n, window);
    const uint32_t nvalid = (len - lo + split - 1) / split;
    const float* part = ws + (uint64_t)unit * nsplit * (D + 2);
    float M = -INFINITY;
    for (uint32_t sp = 0; sp < nvalid; ++sp) M = fmaxf(M, part[sp * (D + 2)]);
    float o = 0.f, l = 0.f;
    for (uint32_t sp = 0; sp < nvalid; ++sp) {
        const float* p = part + sp * (D + 2);
        const float f = fast_exp2(p[0] - M);
        l += f * p[1];
        o += f * p[2 + d];
    }
    const uint32_t s = r / G;
    const uint32_t gh = r - s * G;
    __bf16 hv = (__bf16)(o / l);
    out[(((uint64_t)seq * n + s) * Hq + kvh * G + gh) * D + d] = __builtin_bit_cast(uint16_t, hv);
}

struct SplitPlan {
    uint32_t nsplit, split;
};

// Splits of one view: about kTargetBlocks workgroups in all, whole tiles per
// split.  The workspace stride is the larger full-view plan of the two modes;
// a window plan is capped at the full mixing plan's split count, so it never
// needs a wider stride (rounding splits up to whole tiles can otherwise give
// a shorter window view more splits than the full view).
SplitPlan plan_splits(uint64_t S, uint32_t n, uint32_t Hkv, uint64_t max_tokens, bool within,
                      uint64_t window = 0) {
    const uint64_t units = S * Hkv * (within ? n : 1u);
    auto make = [&](uint64_t len_max, uint64_t cap) -> SplitPlan {
        uint64_t want = (kTargetBlocks + units - 1) / units;
        const uint64_t max_splits = (len_max + DT - 1) / DT;
        if (want > max_splits) want = max_splits;
        if (want > cap) want = cap;
        if (want < 1) want = 1;
        uint64_t split = (len_max + want - 1) / want;
        split = (split + DT - 1) / DT * DT;
        const uint64_t nsplit = (len_max + split - 1) / split;
        return {(uint32_t)nsplit, (uint32_t)split};
    };
    const SplitPlan full = make(within ? max_tokens + 1 : (max_tokens + 1) * n, ~0ull);
    if (within || window == 0 || window + n - 1 >= (max_tokens + 1) * n) return full;
    return make(window + n - 1, full.nsplit);
}

bool decode_sizes_ok(int64_t S, int32_t n, int32_t Hq, int32_t Hkv, int32_t D,
                     int64_t max_tokens) {
    if (S < 0 || n < 1 || Hq < 1 || Hkv < 1 || max_tokens < 0) return false;
    if (Hq % Hkv != 0) return false;
    if (D != 64 && D != 128) return false;
    if ((int64_t)n * (Hq / Hkv) > 64) return false;
    if ((max_tokens + 1) * (int64_t)n > 0x7fffffffLL) return false;
    if (S > 65535) return false;
    return true;
}

}  // namespace

}  // namespace hdsfa

extern "C" size_t sfa_decode_workspace_size(int64_t S, int32_t n, int32_t Hq, int32_t Hkv,
                                            int32_t D, int64_t max_tokens) {
    using namespace hdsfa;
    if (!decode_sizes_ok(S, n, Hq, Hkv, D, max_tokens)) return 0;
    const SplitPlan pw = plan_splits((uint64_t)S, (uint32_t)n, (uint32_t)Hkv, (uint64_t)max_tokens, true);
    const SplitPlan pm = plan_splits((uint64_t)S, (uint32_t)n, (uint32_t)Hkv, (uint64_t)max_tokens, false);
    const uint64_t nsplit = pw.nsplit > pm.nsplit ? pw.nsplit : pm.nsplit;
    const uint64_t R = (uint64_t)n * (Hq / Hkv);
    return (size_t)((uint64_t)S * Hkv * R * nsplit * (uint64_t)(D + 2) * sizeof(float));
}

namespace hdsfa {
namespace {
struct Paging {
    const int32_t* page_table = nullptr;   // nullptr: contiguous [S, C_max, Hkv, D] caches
    uint32_t pshift = 0, mpps = 0, num_pages = 0;
};

// Static scratch of sfa_decode_step_noalloc: the split partials of one call,
// one array per device (each GPU the library runs on holds its own copy until
// the process ends).  Host code never uses the array's name as an address:
// its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// device address of the current device's scratch array (nullptr on failure)
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_status[dev] == hipSuccess ? p : nullptr;
    });
    return g_scratch_status[dev] == hipSuccess ? g_scratch_ptr[dev] : nullptr;
}

// Where the split partials go: the caller's workspace (checked against
// sfa_decode_workspace_size, stride = the larger split count of the two
// modes) or, with use_static, the static scratch (stride = this call's own
// split count, nothing at all when every view is one split).
struct PartialsBuf {
    void* workspace = nullptr;
    size_t workspace_bytes = 0;
    bool use_static = false;
};

hd_status decode_step(const uint16_t* q_new, const uint16_t* k_new, const uint16_t* v_new,
                      uint16_t* k_cache, uint16_t* v_cache, const int32_t* tokens_before,
                      int64_t S, int32_t n, int32_t Hq, int32_t Hkv, int32_t D, int64_t C_max,
                      int64_t max_tokens, int32_t mode, float softmax_scale, const PartialsBuf& pb,
                      uint16_t* out, int32_t* err_flag,
                      hipStream_t stream, int64_t window, const Paging& pg = Paging{}) {
    const bool paged = pg.page_table != nullptr;
    if (S < 0 || n < 1 || Hq < 1 || Hkv < 1 || max_tokens < 0 || C_max < 0) return HD_ERR_SHAPE;
    if (!scale_ok(softmax_scale)) return HD_ERR_SHAPE;
    if (Hq % Hkv != 0) return HD_ERR_SHAPE;
    if (mode != 0 && mode != 1) return HD_ERR_SHAPE;
    if (!decode_sizes_ok(S, n, Hq, Hkv, D, max_tokens)) return HD_ERR_UNSUPPORTED;
    if ((max_tokens + 1) * (int64_t)n > C_max) return HD_ERR_CAPACITY;
    if (S == 0) return HD_OK;
    if (q_new == nullptr || k_new == nullptr || v_new == nullptr || k_cache == nullptr ||
        v_cache == nullptr || tokens_before == nullptr || out == nullptr)
        return HD_ERR_NULL;
    if (!aligned16(q_new) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out))
        return HD_ERR_SHAPE;
    const bool within = mode == 0;
    const uint32_t G = (uint32_t)(Hq / Hkv);
    const uint32_t R = (uint32_t)n * G;
    const uint64_t cache_seq = (uint64_t)C_max * Hkv * D;

    const SplitPlan plan = plan_splits((uint64_t)S, (uint32_t)n, (uint32_t)Hkv, (uint64_t)max_tokens, within,
                                       within ? 0u : (uint64_t)window);
    float* ws = nullptr;
    uint32_t ws_nsplit = 1;
    if (!pb.use_static) {
        const size_t need = sfa_decode_workspace_size(S, n, Hq, Hkv, D, max_tokens);
        if (pb.workspace == nullptr || pb.workspace_bytes < need || !aligned16(pb.workspace))
            return HD_ERR_WORKSPACE;
        // the workspace stride uses the larger plan of the two modes
        const SplitPlan pw = plan_splits((uint64_t)S, (uint32_t)n, (uint32_t)Hkv, (uint64_t)max_tokens, true);
        const SplitPlan pm = plan_splits((uint64_t)S, (uint32_t)n, (uint32_t)Hkv, (uint64_t)max_tokens, false);
        ws_nsplit = pw.nsplit > pm.nsplit ? pw.nsplit : pm.nsplit;
        ws = static_cast<float*>(pb.workspace);
    } else if (plan.nsplit > 1) {
        ws_nsplit = plan.nsplit;
        const uint64_t need = (uint64_t)S * Hkv * R * ws_nsplit * (uint64_t)(D + 2) * sizeof(float);
        if (need > kNoallocScratchBytes) return HD_ERR_SCRATCH;
        ws = static_cast<float*>(scratch_on_current_device());
        if (ws == nullptr) return HD_ERR_LAUNCH;
    }

    // 1. append
    {
        const uint32_t row_chunks = (uint32_t)Hkv * D / 8;
        const uint64_t total = (uint64_t)S * n * row_chunks;
        if (total > 0x7fffffffULL) return HD_ERR_UNSUPPORTED;
        const uint32_t blocks = (uint32_t)((total + 255) / 256);
        (paged ? decode_append_kernel<true> : decode_append_kernel<false>)
            <<<dim3(blocks), dim3(256), 0, stream>>>(
            reinterpret_cast<const u32x4*>(k_new), reinterpret_cast<const u32x4*>(v_new),
            reinterpret_cast<u32x4*>(k_cache), reinterpret_cast<u32x4*>(v_cache),
            tokens_before, (uint32_t)S, (uint32_t)n, row_chunks, cache_seq / 8,
            (uint32_t)max_tokens, pg.page_table, pg.pshift, pg.mpps, pg.num_pages, err_flag);
        const hd_status st = launch_status();
        if (st != HD_OK) return st;
    }

    // 2. attend
    DecodeArgs a;
    a.q = q_new;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tokens_before = tokens_before;
    a.ws = ws;
    a.cache_seq = cache_seq;
    a.n = (uint32_t)n;
    a.Hq = (uint32_t)Hq;
    a.Hkv = (uint32_t)Hkv;
    a.G = G;
    a.R = R;
    a.max_tokens = (uint32_t)max_tokens;
    a.nsplit = ws_nsplit;
    a.split = plan.split;
    a.within = within ? 1u : 0u;
    a.window = within ? 0u : (uint32_t)window;
    a.c = softmax_scale * kLog2e;
    a.page_table = pg.page_table;
    a.pshift = pg.pshift;
    a.mpps = pg.mpps;
    a.num_pages = pg.num_pages;
    a.out = out;
    a.direct = plan.nsplit == 1 ? 1u : 0u;
    a.err = err_flag;
    const uint32_t rows = within ? G : R;
    const dim3 grid(plan.nsplit, (uint32_t)Hkv * (within ? (uint32_t)n : 1u), (uint32_t)S);
    if (D == 128) {
        if (rows <= 32) (paged ? decode_attend_kernel<128, 1, true> : decode_attend_kernel<128, 1, false>)
                            <<<grid, dim3(DTHREADS), 0, stream>>>(a);
        else            (paged ? decode_attend_kernel<128, 2, true> : decode_attend_kernel<128, 2, false>)
                            <<<grid, dim3(DTHREADS), 0, stream>>>(a);
    } else {
        if (rows <= 32) (paged ? decode_attend_kernel<64, 1, true> : decode_attend_kernel<64, 1, false>)
                            <<<grid, dim3(DTHREADS), 0, stream>>>(a);
        else            (paged ? decode_attend_kernel<64, 2, true> : decode_attend_kernel<64, 2, false>)
                            <<<grid, dim3(DTHREADS), 0, stream>>>(a);
    }
    hd_status st = launch_status();
    if (st != HD_OK) return st;
    if (a.direct) return HD_OK;

    // 3. combine (more than one split per view)
    const uint64_t total = (uint64_t)S * Hkv * R * D;
    if (total > 0x7fffffffULL) return HD_ERR_UNSUPPORTED;
    const uint32_t blocks = (uint32_t)((total + 255) / 256);
    if (D == 128)
        decode_combine_kernel<128><<<dim3(blocks), dim3(256), 0, stream>>>(
            a.ws, tokens_before, out, (uint32_t)S, (uint32_t)n, (uint32_t)Hq, (uint32_t)Hkv, G, R,
            ws_nsplit, plan.split, a.within, (uint32_t)max_tokens, a.window);
    else
        decode_combine_kernel<64><<<dim3(blocks), dim3(256), 0, stream>>>(
            a.ws, tokens_before, out, (uint32_t)S, (uint32_t)n, (uint32_t)Hq, (uint32_t)Hkv, G, R,
            ws_nsplit, plan.split, a.within, (uint32_t)max_tokens, a.window);
    return launch_status();
}
}  // namespace
}  // namespace hdsfa

extern "C" hd_status sfa_decode_step(const uint16_t* q_new, const uint16_t* k_new,
                                     const uint16_t* v_new, uint16_t* k_cache,
                                     uint16_t* v_cache, const int32_t* tokens_before,
                                     int64_t S, int32_t n, int32_t Hq, int32_t Hkv,
                                     int32_t D, int64_t C_max, int64_t max_tokens,
                                     int32_t mode, float softmax_scale, void* workspace,
                                     size_t workspace_bytes, uint16_t* out,
                                     int32_t* err_flag, hipStream_t stream) {
    hdsfa::PartialsBuf pb;
    pb.workspace = workspace;
    pb.workspace_bytes = workspace_bytes;
    return hdsfa::decode_step(q_new, k_new, v_new, k_cache, v_cache, tokens_before, S, n, Hq, Hkv, D,
                              C_max, max_tokens, mode, softmax_scale, pb, out, err_flag, stream, 0);
}

extern "C" hd_status sfa_decode_step_noalloc(const uint16_t* q_new, const uint16_t* k_new,
                                             const uint16_t* v_new, uint16_t* k_cache,
                                             uint16_t* v_cache, const int32_t* tokens_before,
                                             int64_t S, int32_t n, int32_t Hq, int32_t Hkv,
                                             int32_t D, int64_t C_max, int64_t max_tokens,
                                             int32_t mode, float softmax_scale, uint16_t* out,
                                             int32_t* err_flag, hipStream_t stream) {
    hdsfa::PartialsBuf pb;
    pb.use_static = true;
    return hdsfa::decode_step(q_new, k_new, v_new, k_cache, v_cache, tokens_before, S, n, Hq, Hkv, D,
                              C_max, max_tokens, mode, softmax_scale, pb, out, err_flag, stream, 0);
}

extern "C" hd_status sfa_decode_step_paged(const uint16_t* q_new, const uint16_t* k_new,
                                           const uint16_t* v_new, uint16_t* k_pages,
                                           uint16_t* v_pages, const int32_t* page_table,
                                           const int32_t* tokens_before, int64_t S, int32_t n,
                                           int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                           int64_t num_pages, int32_t max_pages_per_seq,
                                           int64_t max_tokens, int32_t mode, int64_t window,
                                           float softmax_scale, void* workspace,
                                           size_t workspace_bytes, uint16_t* out,
                                           int32_t* err_flag, hipStream_t stream) {
    using namespace hdsfa;
    if (page_size < 1 || (page_size & (page_size - 1)) != 0) return HD_ERR_SHAPE;
    if (num_pages < 1 || num_pages > 0x7fffffffLL || max_pages_per_seq < 1) return HD_ERR_SHAPE;
    // pool row indices are 32-bit on the device
    if ((uint64_t)num_pages * (uint64_t)page_size > 0x100000000ULL) return HD_ERR_UNSUPPORTED;
    if (window < 0 || (window > 0 && mode != 1) || window > 0x7fffffffLL) return HD_ERR_SHAPE;
    if (S > 0 && page_table == nullptr) return HD_ERR_NULL;
    Paging pg;
    pg.page_table = page_table;
    pg.pshift = (uint32_t)__builtin_ctz((unsigned)page_size);
    pg.mpps = (uint32_t)max_pages_per_seq;
    pg.num_pages = (uint32_t)num_pages;
    const int64_t capacity = (int64_t)max_pages_per_seq * page_size;   // entries a sequence can hold
    if (S == 0) pg.page_table = nullptr;
    PartialsBuf pb;
    pb.workspace = workspace;
    pb.workspace_bytes = workspace_bytes;
    return decode_step(q_new, k_new, v_new, k_pages, v_pages, tokens_before, S, n, Hq, Hkv, D,
                       capacity, max_tokens, mode, softmax_scale, pb, out, err_flag, stream, window, pg);
}

extern "C" hd_status sfa_decode_step_window(const uint16_t* q_new, const uint16_t* k_new,
                                            const uint16_t* v_new, uint16_t* k_cache,
                                            uint16_t* v_cache, const int32_t* tokens_before,
                                            int64_t S, int32_t n, int32_t Hq, int32_t Hkv,
                                            int32_t D, int64_t C_max, int64_t max_tokens,
                                            int64_t window, float softmax_scale, void* workspace,
                                            size_t workspace_bytes, uint16_t* out,
                                            int32_t* err_flag, hipStream_t stream) {
    if (window < 1 || window > 0x7fffffffLL) return HD_ERR_SHAPE;
    hdsfa::PartialsBuf pb;
    pb.workspace = workspace;
    pb.workspace_bytes = workspace_bytes;
    return hdsfa::decode_step(q_new, k_new, v_new, k_cache, v_cache, tokens_before, S, n, Hq, Hkv, D,
                              C_max, max_tokens, 1, softmax_scale, pb, out, err_flag, stream, window);
}

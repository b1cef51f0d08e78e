// Stream-Factorized Attention, prefill (sfa_stream_attn, sfa_mix_attn,
// sfa_mix_attn_window, and the training forwards sfa_attn_fwd and
// sfa_attn_fwd_window, which also write each row's log-sum-exp).
//
// "Hidden Decoding at Scale" review, section Method: in the majority of layers a
// position sees only its own stream (cost of order n*L^2); the few others let
// streams see each other with the base model's full causal pattern over the
// length-nL sequence.  The arXiv 2607.08186 abstract: so the attention cost
// grows about linearly with n rather than with its square.
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
// A sliding-window mixing layer (the base model's windowed pattern) is the
// mixing view with a lower bound: query i sees keys j with i - W < j <= i
// (W in expanded positions).  An item then starts at the key tile holding its
// first row's oldest visible key, and the rows' lower bounds are masked on the
// one or two tiles they cross.
//
// Work items are (query tile, batch, view, KV head, head pack), listed longest
// causal extent first.  The grid is persistent, one workgroup per compute
// unit (HD_SFA_PREFILL_WORKGROUPS in the environment sets another count):
// workgroup b takes item r*grid + b on even rounds r and r*grid + (grid-1-b)
// on odd rounds, which evens out the triangular costs.
// While a workgroup normalises and stores one item's output, the Q fragments
// and first K/V tiles of its next item are already on their way.
//
// Workgroup = 8 waves (2 per SIMD).  Each wave owns 32 query rows of one query
// head and computes S^T = K Q^T and O^T += V^T P^T with the gfx950 bf16 matrix
// op v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  Keeping S transposed puts
// one query per lane (pair of lanes), so row max / row sum are per-lane values
// plus one exchange with the other half-wave, and the probabilities leave the
// accumulator already in the B-operand layout of the second product.
// GQA: the query heads sharing a KV head are packed into one workgroup so each
// K/V tile is staged once in LDS for all of them.
//
// K and V tiles of 64 keys are copied global -> LDS by direct loads
// (global_load_lds, 16 bytes per lane) into a two-deep ring, row-major with an
// XOR swizzle of the 16-byte chunks.  K fragments are 16-byte LDS reads; the
// V^T operand comes from transpose reads (ds_read_b64_tr_b16).
//
// Per key tile a wave runs two phases: the online softmax (vector ALU) and
// the matrix phase (the score product of the next tile and the value product
// of this one).  The matrix phase is generated assembly (prefill_asm.h) that
// issues every LDS operand read several MFMAs ahead of its use; the two waves
// that share a SIMD run the phases half a tile apart, so one wave's softmax
// overlaps the other's matrix products.
#include "common.h"
#include "prefill_asm.h"

#include <algorithm>
#include <cstdlib>
#include <type_traits>

namespace hdsfa {

namespace {

constexpr int BN = 64;       // keys per tile
constexpr int MQ = 32;       // query rows per wave
constexpr int NW = 8;        // waves per workgroup (2 per SIMD)
constexpr int NSTAGE = 2;    // LDS ring depth for K and for V tiles
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
    uint32_t n_items;    // n_qtiles * B * groups * Hkv * n_hpacks
    uint32_t window;     // sliding window W in rows of the view (WIN kernels only)
    float c;             // softmax scale * log2(e)
    float* lse;          // optional [B, Hq, N] natural log-sum-exp of each row (training)
    uint32_t Hq, N;
    // key-split launches (SPLIT kernels only): units n_items + n_split, see
    // make_item; per (item, wave) a counter and two partial-state slots
    uint32_t n_units;
    uint32_t n_split;    // items with two or more key tiles (a prefix of the item order)
    uint32_t* cnt;       // [n_split * NW], zero between calls
    float* part;         // [n_split, 2, NW, slot floats]
};

// Scale modes: the exponent argument of a score s is s * c - m with
// c = softmax scale * log2(e).
//   kScaleAny:  c from the arguments (v_fma_f32, 8-byte encoding);
//   kScaleUnit: scale 1 (Q carries the softmax scale), c = log2(e) is a literal
//               (v_fmamk_f32, 8 bytes);
//   kScaleLog2: c == 1 (Q also carries log2(e): scores arrive in log2 units),
//               the argument is s - m (v_add_f32, 4 bytes).
// The softmax issue time of a wave is close to proportional to its
// instruction bytes, so the shorter form matters.
constexpr int kScaleAny = 0, kScaleUnit = 1, kScaleLog2 = 2;
// Floats of one wave's partial softmax state in a key-split launch: per lane
// its O^T accumulators (D/32 blocks of 16) and (m, l).
template <int D>
constexpr int split_slot_floats() { return kWave * (D / 2 + 2); }

// WIN: sliding window (a.window < len); otherwise plain causal.
// SPLIT: key-split launch (no window): an item with two or more key tiles is
// taken as two units, its first and second half of the tiles, by different
// workgroups; each writes its partial softmax state (m, l, O) and the second
// to finish merges both and writes the output.
template <int D, int MODE, bool WIN, bool SPLIT>
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
sfa_prefill_kernel(const PrefillArgs a) {
    static_assert(!(WIN && SPLIT), "a windowed layer is not key-split");
    constexpr int ROWB = D * 2;                // bytes per K/V row
    constexpr int TILE_B = BN * ROWB;          // one K (or V) tile
    constexpr int LOADS = TILE_B / (THREADS * 16);   // 16-byte direct loads per thread per tile
    constexpr int DSTEPS = D / 16;             // k-steps of the score product
    constexpr int DBLK = D / 32;               // 32-row blocks of O^T
    static_assert(TILE_B % (THREADS * 16) == 0, "tile/thread mismatch");

    constexpr int QW_B = DSTEPS * 1024;        // one wave's Q fragments
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * NSTAGE * TILE_B + NW * QW_B];   // K ring, V ring, Q

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;                  // half-wave index
    // the lane index through an opaque copy: address arithmetic derived from
    // it in code that runs once per item is computed where it is used instead
    // of being hoisted out of the key loop and held in registers
    auto lane_here = [&]() __attribute__((always_inline)) -> uint32_t {
        uint32_t v;
        asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"((uint32_t)lane));
        return v;
    };

    const int qblocks = NW / a.P;
    const uint32_t BT = MQ * qblocks;          // query rows per work item
    const uint32_t per_tile = a.B * a.groups * a.Hkv * a.n_hpacks;

    bf16x8 qf[DSTEPS];                         // Q fragments of the current item
    f32x16 oacc[DBLK];                         // O^T accumulators
    float m_run, l_run;   // running max (log2 units, already * c) and sum of exp2

    // ---- work items ----
    // Only what the key loop needs stays live across an item (the views, the
    // tile counts and the lane's query row); the Q and O row addresses are
    // recomputed from the item index where they are used.
    struct Item {
        uint32_t id;          // the item (a key-split unit's item)
        const char* kview;
        const char* vview;
        int n_kt;             // end of the unit's key tiles (absolute; the item's end unless split)
        int wave_kt;          // key tiles this wave needs (absolute end)
        int m_lo;             // first key tile of the unit (0 without a window or split)
        int wave_lo;          // this wave's first key tile
        int lo_end;           // last tile holding a key below some row's window (-1: none)
        uint32_t qi;          // this lane's query row in the view
        int part;             // key-split: -1 whole item, else 0 / 1 (first / second half)
    };
    // (batch, view, query head) offset of an item, in elements, and its first row
    auto item_head = [&](uint32_t id, uint32_t& q0) -> uint64_t {
        const uint32_t qtile = a.n_qtiles - 1 - id / per_tile;
        id %= per_tile;
        const uint32_t hp = id % a.n_hpacks;
        id /= a.n_hpacks;
        const uint32_t kvh = id % a.Hkv;
        id /= a.Hkv;
        const uint32_t grp = id % a.groups;
        const uint32_t b = id / a.groups;
        q0 = qtile * BT + (wave / a.P) * MQ;
        return b * a.q_batch + grp * a.q_group + (uint64_t)(kvh * a.G + hp * a.P + (wave % a.P)) * D;
    };
    auto make_item = [&](uint32_t unit) -> Item {
        Item it;
        // key-split units: n_items first halves (whole items when they have
        // one tile), then the second halves of the first n_split items
        const uint32_t id = (SPLIT && unit >= a.n_items) ? unit - a.n_items : unit;
        it.id = id;
        const uint32_t qtile = a.n_qtiles - 1 - id / per_tile;
        uint32_t r = id % per_tile;
        r /= a.n_hpacks;
        const uint32_t kvh = r % a.Hkv;
        r /= a.Hkv;
        const uint32_t grp = r % a.groups;
        const uint32_t b = r / a.groups;
        it.kview = reinterpret_cast<const char*>(a.k + b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D);
        it.vview = reinterpret_cast<const char*>(a.v + b * a.kv_batch + grp * a.kv_group + (uint64_t)kvh * D);
        const uint32_t wg_end = min(a.len, (qtile + 1) * BT);
        it.n_kt = (int)((wg_end + BN - 1) / BN);
        const uint32_t q0 = qtile * BT + (wave / a.P) * MQ;
        const uint32_t wave_end = min(a.len, q0 + MQ);       // exclusive
        it.wave_kt = q0 < a.len ? (int)((wave_end + BN - 1) / BN) : 0;
        it.qi = q0 + l32;
        it.part = -1;
        if constexpr (WIN) {
            // oldest visible key of row r: r - W + 1 (clamped at 0)
            const uint32_t f0 = qtile * BT;
            it.m_lo = (int)((f0 >= a.window ? f0 - a.window + 1 : 0u) / BN);
            it.wave_lo = (int)((q0 >= a.window ? q0 - a.window + 1 : 0u) / BN);
            it.lo_end = q0 + MQ - 1 >= a.window ? (int)((q0 + MQ - 1 - a.window) / BN) : -1;
        } else {
            it.m_lo = 0;
            it.wave_lo = 0;
            it.lo_end = -1;
            if constexpr (SPLIT) {
                if (it.n_kt >= 2) {
                    const int half = (it.n_kt + 1) / 2;
                    if (unit < a.n_items) {
                        it.part = 0;
                        it.n_kt = half;
                    } else {
                        it.part = 1;
                        it.m_lo = half;
                    }
                }
            }
        }
        return it;
    };
    // first tiles (window or key split); compile-time zero otherwise
    auto lo_of = [&](const Item& it) -> int { if constexpr (WIN || SPLIT) return it.m_lo; else return 0; };
    auto wlo_of = [&](const Item& it) -> int {
        if constexpr (WIN) return it.wave_lo;
        else if constexpr (SPLIT) return it.m_lo;    // every wave starts at the unit's first tile
        else return 0;
    };
    // item taken in round r (snake order over the grid)
    auto item_at = [&](uint32_t r) -> uint32_t {
        const uint32_t g = gridDim.x;
        return r * g + ((r & 1u) ? (g - 1u - blockIdx.x) : blockIdx.x);   // a unit in key-split launches
    };

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
    auto kbuf = [&](int t) { return smem + (t & 1) * TILE_B; };
    auto vbuf = [&](int t) { return smem + (NSTAGE + (t & 1)) * TILE_B; };
    // Q of an item, global -> this wave's LDS Q area (its 32 rows), stored
    // like a K tile: row-major with the XOR swizzle of the 16-byte chunks, so
    // that every load instruction reads whole rows (4 rows of 256 bytes at
    // head_dim 128) and the fragments are read back as the K operands are.
    // Rows past the view end are clamped into it and never stored.  The
    // area is read once at the start of the item, so the next item's Q can
    // be requested any time after that.
    unsigned char* const qlds = smem + 2 * NSTAGE * TILE_B + wave * QW_B;
    auto issue_q = [&](uint32_t id) {
        constexpr uint32_t CPR = ROWB / 16;    // 16-byte chunks per row
        constexpr uint32_t RPL = 1024 / ROWB;  // rows per load instruction
        static_assert(MQ / RPL == DSTEPS && MQ * ROWB == QW_B, "Q area layout");
        const uint32_t ln = lane_here();
        uint32_t q0;
        const uint64_t hoff = item_head(id, q0);
        const char* base = reinterpret_cast<const char*>(a.q + hoff);
        const uint32_t j = ln / CPR, p = ln % CPR;
#pragma unroll
        for (uint32_t e = 0; e < (uint32_t)MQ / RPL; ++e) {
            const uint32_t row = e * RPL + j;
            const uint64_t qrow = min(q0 + row, a.len - 1u);
            const char* src = base + qrow * (a.q_row * 2u) + ((p ^ swz<D>(row)) << 4);
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)src,
                (void __attribute__((address_space(3)))*)(qlds + e * 1024), 16, 0, 0);
        }
    };

    // ---- output ----
    // O = O^T / l leaves through 2 KB per wave of V slot 1, which no wave
    // reads or fills between the barrier that ends an item and the first step
    // of the next: per 32-dim block the wave writes its 32 rows x 64 bytes
    // (16-byte chunks XOR-swizzled by row), reads them back 4 lanes per row,
    // and stores whole 64-byte row pieces.
    auto store_out = [&](uint32_t id, uint32_t qi) {
        const uint32_t ln = lane_here(), r32 = ln & 31u, h2 = ln >> 5;
        uint32_t q0;
        uint16_t* obase = a.o + item_head(id, q0);
        const float inv = 1.f / l_run;         // unused (never stored) where qi >= len
        if constexpr (TILE_B >= NW * 2048) {
            unsigned char* stg = vbuf(1) + wave * 2048;
            const uint32_t rr = ln >> 2, rc = ln & 3u;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x2 w = {pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                                     pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                    const uint32_t pc = (uint32_t)g ^ ((r32 >> 2) & 3u);
                    *reinterpret_cast<u32x2*>(stg + r32 * 64 + pc * 16 + h2 * 8) = w;
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t r = rr + 16u * h;
                    const u32x4 w = *reinterpret_cast<const u32x4*>(stg + r * 64 + ((rc ^ ((r >> 2) & 3u)) << 4));
                    if (q0 + r < a.len)
                        *reinterpret_cast<u32x4*>(obase + (uint64_t)(q0 + r) * a.q_row + db * 32 + rc * 8) = w;
                }
            }
        } else if (qi < a.len) {
            // 4 consecutive dims per lane and item group
            uint16_t* orow = obase + (uint64_t)qi * a.q_row;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + 8 * g + 4 * (int)h2;
                    u32x2 w = {pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                               pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2*>(orow + d) = w;
                }
        }
    };

    // ---- key-split units ----
    // A unit's wave writes its partial state (its O^T accumulators, m and l,
    // which are in log2 units relative to m) to its slot, then counts itself
    // in the (item, wave) counter.  The wave that counts second has both
    // states: it merges them into its registers, writes the output and
    // clears the counter for the next call; the other one is done.  Neither
    // waits for the other.  The slots are written and read with device-scope
    // accesses (they bypass the compute unit's and its XCD's caches where
    // those are not coherent across the device), and the writes have
    // completed before the count is taken, so the wave that counts second
    // reads the other state whole; no cache-wide write-back or invalidation
    // is needed.  The merge takes both products explicitly (no contraction),
    // so it gives the same bits whichever half merges.
    auto merge_split = [&](const Item& it) -> bool {
        constexpr int SF = split_slot_floats<D>();
        constexpr int OFL = DBLK * 16 * kWave;     // floats of the accumulators in a slot
        const uint32_t w = __builtin_amdgcn_readfirstlane(wave);
        float* const slots = a.part + (size_t)it.id * 2 * NW * SF;
        uint64_t* const own = reinterpret_cast<uint64_t*>(slots + (size_t)(it.part * NW + w) * SF);
        uint64_t* const oth = reinterpret_cast<uint64_t*>(slots + (size_t)((it.part ^ 1) * NW + w) * SF);
        auto pack2 = [](float lo, float hi) -> uint64_t {
            return (uint64_t)__builtin_bit_cast(uint32_t, lo) | ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
        };
        auto lo_of2 = [](uint64_t x) { return __builtin_bit_cast(float, (uint32_t)x); };
        auto hi_of2 = [](uint64_t x) { return __builtin_bit_cast(float, (uint32_t)(x >> 32)); };
        // pair k of accumulator block db at (db * 8 + k) * 64 + lane (8-byte units)
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int k2 = 0; k2 < 8; ++k2)
                __hip_atomic_store(own + (db * 8 + k2) * kWave + lane,
                                   pack2(oacc[db][2 * k2], oacc[db][2 * k2 + 1]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(own + OFL / 2 + lane, pack2(m_run, l_run), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the state is written before it counts
        uint32_t old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(a.cnt + (size_t)it.id * NW + w, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old == 0) return false;
        const uint64_t ml = __hip_atomic_load(oth + OFL / 2 + lane, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
        {
#pragma clang fp contract(off)
            const float mo = lo_of2(ml);
            const float mn = fmaxf(m_run, mo);
            const float sw = fast_exp2(m_run - mn), so = fast_exp2(mo - mn);
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
#pragma unroll
                for (int k2 = 0; k2 < 8; ++k2) {
                    const uint64_t x = __hip_atomic_load(oth + (db * 8 + k2) * kWave + lane,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    oacc[db][2 * k2] = oacc[db][2 * k2] * sw + lo_of2(x) * so;
                    oacc[db][2 * k2 + 1] = oacc[db][2 * k2 + 1] * sw + hi_of2(x) * so;
                }
            }
            l_run = l_run * sw + hi_of2(ml) * so;
            m_run = mn;
        }
        if (lane == 0)
            __hip_atomic_store(a.cnt + (size_t)it.id * NW + w, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        return true;
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


    // online softmax of one tile's scores; returns the P^T operands.  The
    // causal mask is needed only on a wave's last (diagonal) tile.
    //
    // Lazy rescale: the reference max m_run only moves when a row's tile max
    // exceeds it by more than 8 (a factor 2^8), so O and l are rescaled
    // rarely (always on the first tile).  Probabilities stay <= 2^8 and the
    // result O / l is unchanged.  Away from the first and the diagonal tile
    // the tile max is not computed at all: the exponentials are taken with the
    // current m_run, and if no row's tile sum exceeds 2^8 then no p exceeds
    // 2^8, so no row's max exceeds m_run + 8 and the max test would not have
    // rescaled either.  Only when a row's sum exceeds 2^8 (rare once the max
    // has settled) are the max test and the exponentials done again, which
    // gives exactly the result of always testing the max.
    auto softmax = [&](f32x16 (&sacc)[BN / 32], int kt, bool diag, bool lowmask, bool first,
                       uint32_t qi, bf16x8 (&pf)[BN / 16]) {
        // item (kb, it) holds key kt*BN + off + 4*hh with off = kb*32 + 8*(it/4)
        // + it%4 (0..63, an inline constant): each mask is one compare of off
        // against a per-lane threshold
        const int rel = (int)qi - kt * BN - 4 * hh;
        if (diag) {
            // keys later than the query
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int it = 0; it < 16; ++it) {
                    const int off = kb * 32 + 8 * (it >> 2) + (it & 3);
                    if (off > rel) sacc[kb][it] = -INFINITY;
                }
        }
        if (WIN && lowmask) {
            // keys at or below qi - W are outside the row's window
            const int lim = rel - (int)a.window;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int it = 0; it < 16; ++it) {
                    const int off = kb * 32 + 8 * (it >> 2) + (it & 3);
                    if (off <= lim) sacc[kb][it] = -INFINITY;
                }
        }
        auto max_test = [&]() __attribute__((always_inline)) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int it = 0; it < 16; ++it) mx = fmaxf(mx, sacc[kb][it]);
            if constexpr (MODE == kScaleUnit) mx = halves_max(mx) * kLog2e;
            else if constexpr (MODE == kScaleAny) mx = halves_max(mx) * a.c;
            else mx = halves_max(mx);
            if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.f) != 0) {
                const float m_new = fmaxf(m_run, mx);
                // a windowed row may have seen no visible key yet (m_new = -inf)
                const float alpha = (WIN && m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < DBLK; ++i) oacc[i] *= alpha;
            }
        };
        // p = 2^(s*c - m_run) into the P^T fragments (16-key step c takes
        // items 8*(c%2)..+7); returns the row's tile sum.  S is left intact.
        auto exps = [&]() __attribute__((always_inline)) -> float {
            // -m in a register of its own (not a negate modifier), so that the
            // exponent argument has a two-operand form (v_fmamk_f32 / v_add_f32)
            float nm;
            asm("v_xor_b32 %0, 0x80000000, %1" : "=v"(nm) : "v"(m_run));
            if constexpr (WIN) nm = m_run == -INFINITY ? 0.f : nm;   // such a row has only masked scores
            float rsp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < BN / 16; ++c) {
                const f32x16& sv = sacc[c >> 1];
                const int o8 = (c & 1) * 8;
                f32x8 pv;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float x;
                    if constexpr (MODE == kScaleLog2) x = sv[o8 + j] + nm;
                    else x = __builtin_fmaf(sv[o8 + j], MODE == kScaleUnit ? kLog2e : a.c, nm);
                    pv[j] = fast_exp2(x);
                    rsp[j & 3] += pv[j];
                }
                pf[c] = to_bf16x8(pv);
            }
            return halves_sum((rsp[0] + rsp[1]) + (rsp[2] + rsp[3]));
        };
        float ts;
        if (diag || first) {
            max_test();
            ts = exps();
        } else {
            ts = exps();
            // with a window, a row that has seen no visible key yet still has
            // m_run = -inf, which cannot serve as the reference: retry too
            bool retry = ts > 256.f;
            if constexpr (WIN) retry = retry || m_run == -INFINITY;
            if (__builtin_amdgcn_ballot_w64(retry) != 0) {
                max_test();
                ts = exps();
            }
        }
        l_run += ts;
    };

    // ---- software pipeline over key tiles ----
    // Two phases per key tile m:
    //   A(m): online softmax of S(m) into P(m) (VALU);
    //   B(m): S(m+1) = K(m+1) Q^T and O^T += V(m)^T P(m)^T (32 MFMAs at
    //         head_dim 128, LDS operands read ahead; generated assembly).
    // The two waves sharing a SIMD run them half a step apart: waves 0-3 do
    // A(m), barrier, B(m); waves 4-7 do barrier, A(m), B(m) ... so one wave's
    // softmax overlaps the other's matrix products.  Barrier m (one per key
    // tile, reached by every wave) orders the LDS ring: both groups read
    // K(m+1) and V(m) between barriers m and m+1, so at barrier m the slots of
    // K(m) and V(m-1) are free and receive K(m+2) and V(m+1), waited for at
    // barrier m+1.  In the final interval F no K tile is read and only V(F):
    // there the next item's Q, K(0), K(1) and, if its slot is free (F odd),
    // V(0) are requested.
    const int wgrp = __builtin_amdgcn_readfirstlane(wave) >> 2;   // one wave of each group per SIMD
    f32x16 sc[BN / 32];                        // S(m) (scores), then P(m) in place
    bf16x8 pf[BN / 16];                        // P(m) as B operands of the value product
    const uint32_t lds0 = lds_addr(smem);
    uint32_t KA[DSTEPS], VA[2 * DBLK];         // LDS addresses of this lane's K / V reads
#pragma unroll
    for (int e = 0; e < DSTEPS; ++e) KA[e] = lds0 + koff[e];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int db = 0; db < DBLK; ++db) VA[rd * DBLK + db] = lds0 + voff[rd][db];

    // steps are counted from the item's first tile: r = m - m_lo picks the
    // ring slots, m addresses the view
    auto barrier_step = [&](int r, const Item& cur, uint32_t nid, bool more) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int m = lo_of(cur) + r;
        if (m + 2 < cur.n_kt) issue(cur.kview, m + 2, kbuf(r + 2));
        if (m + 1 < cur.n_kt) issue(cur.vview, m + 1, vbuf(r + 1));
        if (m == cur.n_kt - 1 && more) {
            // an opaque copy of the index keeps the address arithmetic here
            // (it is loop-invariant) from being hoisted and held in registers
            // across the whole key loop
            uint32_t id2;
            asm volatile("s_mov_b32 %0, %1" : "=s"(id2) : "s"(nid));
            const Item nx = make_item(id2);
            issue_q(nx.id);                    // the unit's item
            issue(nx.kview, lo_of(nx), kbuf(0));
            if (lo_of(nx) + 1 < nx.n_kt) issue(nx.kview, lo_of(nx) + 1, kbuf(1));
            if (r & 1) issue(nx.vview, lo_of(nx), vbuf(0));
        }
    };
    auto phase_a = [&](int r, const Item& cur) {
        const int m = lo_of(cur) + r;
        const int last = cur.wave_kt - 1;      // the wave's diagonal tile takes the mask
        if (m >= wlo_of(cur) && m <= last)
            softmax(sc, m, m == last, WIN && m <= cur.lo_end, m == wlo_of(cur), cur.qi, pf);
    };
    // B(m) with m of parity PAR (fixes the LDS slots of K(m+1) and V(m))
    auto phase_b = [&](auto par, int r, const Item& cur) {
        constexpr int PAR = decltype(par)::value;
        const int m = lo_of(cur) + r;
        const int last = cur.wave_kt - 1;
        f32x16(&S)[BN / 32] = sc;
        f32x16(&O)[DBLK] = oacc;
        const bf16x8(&Q)[DSTEPS] = qf;
        const bf16x8(&P)[BN / 16] = pf;
        // a wave computes P(m) for wave_lo <= m <= last and S(m+1) when m+1 is
        // in that range too (without a window wave_lo = 0)
        const bool do_pv = m >= wlo_of(cur) && m <= last;
        const bool do_qk = m + 1 >= wlo_of(cur) && m < last && (!SPLIT || m + 1 < cur.n_kt);
        if (do_pv && do_qk) {
            if constexpr (D == 128) {
                if constexpr (PAR == 0) asm volatile(HD_ASM_FULL_D128_P0 : HD_ASM_OUTS_FULL_D128 : HD_ASM_INS_FULL_D128 : HD_ASM_CLOBBERS);
                else asm volatile(HD_ASM_FULL_D128_P1 : HD_ASM_OUTS_FULL_D128 : HD_ASM_INS_FULL_D128 : HD_ASM_CLOBBERS);
            } else {
                if constexpr (PAR == 0) asm volatile(HD_ASM_FULL_D64_P0 : HD_ASM_OUTS_FULL_D64 : HD_ASM_INS_FULL_D64 : HD_ASM_CLOBBERS);
                else asm volatile(HD_ASM_FULL_D64_P1 : HD_ASM_OUTS_FULL_D64 : HD_ASM_INS_FULL_D64 : HD_ASM_CLOBBERS);
            }
        } else if (do_pv) {
            if constexpr (D == 128) {
                if constexpr (PAR == 0) asm volatile(HD_ASM_PV_D128_P0 : HD_ASM_OUTS_PV_D128 : HD_ASM_INS_PV_D128 : HD_ASM_CLOBBERS);
                else asm volatile(HD_ASM_PV_D128_P1 : HD_ASM_OUTS_PV_D128 : HD_ASM_INS_PV_D128 : HD_ASM_CLOBBERS);
            } else {
                if constexpr (PAR == 0) asm volatile(HD_ASM_PV_D64_P0 : HD_ASM_OUTS_PV_D64 : HD_ASM_INS_PV_D64 : HD_ASM_CLOBBERS);
                else asm volatile(HD_ASM_PV_D64_P1 : HD_ASM_OUTS_PV_D64 : HD_ASM_INS_PV_D64 : HD_ASM_CLOBBERS);
            }
        } else if (WIN && do_qk) {
            // the tile before this wave's first one: only the scores of the next
            if constexpr (D == 128) {
                if constexpr (PAR == 0) asm volatile(HD_ASM_QK_D128_P0 : HD_ASM_OUTS_QK_D128 : HD_ASM_INS_QK_D128 : HD_ASM_CLOBBERS);
                else asm volatile(HD_ASM_QK_D128_P1 : HD_ASM_OUTS_QK_D128 : HD_ASM_INS_QK_D128 : HD_ASM_CLOBBERS);
            } else {
                if constexpr (PAR == 0) asm volatile(HD_ASM_QK_D64_P0 : HD_ASM_OUTS_QK_D64 : HD_ASM_INS_QK_D64 : HD_ASM_CLOBBERS);
                else asm volatile(HD_ASM_QK_D64_P1 : HD_ASM_OUTS_QK_D64 : HD_ASM_INS_QK_D64 : HD_ASM_CLOBBERS);
            }
        }
    };
    auto step = [&](auto par, int r, const Item& cur, uint32_t nid, bool more) {
        if (wgrp) barrier_step(r, cur, nid, more);
        phase_a(r, cur);
        if (!wgrp) barrier_step(r, cur, nid, more);
        phase_b(par, r, cur);
    };

    // ---- persistent loop over this workgroup's work items ----
    uint32_t round = 0;
    const uint32_t first = item_at(0);
    if (first >= a.n_units) return;            // uniform over the workgroup
    Item cur = make_item(first);
    issue_q(cur.id);
    issue(cur.kview, lo_of(cur), kbuf(0));
    issue(cur.vview, lo_of(cur), vbuf(0));
    if (lo_of(cur) + 1 < cur.n_kt) issue(cur.kview, lo_of(cur) + 1, kbuf(1));
    for (;;) {
        const uint32_t nid = item_at(round + 1);
        const bool more = nid < a.n_units;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int e = 0; e < DSTEPS; ++e)
            qf[e] = *reinterpret_cast<const bf16x8*>(qlds + koff[e]);   // row l32, chunk 2e + hh
#pragma unroll
        for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
        m_run = -INFINITY;
        l_run = 0.f;
        if (cur.wave_kt > lo_of(cur)) {
            // S of the item's first tile (K slot 0: the score product of parity 1)
            f32x16(&S)[BN / 32] = sc;
            const bf16x8(&Q)[DSTEPS] = qf;
            if constexpr (D == 128) asm volatile(HD_ASM_QK_D128_P1 : HD_ASM_OUTS_QK_D128 : HD_ASM_INS_QK_D128 : HD_ASM_CLOBBERS);
            else asm volatile(HD_ASM_QK_D64_P1 : HD_ASM_OUTS_QK_D64 : HD_ASM_INS_QK_D64 : HD_ASM_CLOBBERS);
        }
        const int steps = cur.n_kt - lo_of(cur);
        for (int r = 0; r < steps; r += 2) {
            step(std::integral_constant<int, 0>{}, r, cur, nid, more);
            if (r + 1 < steps) step(std::integral_constant<int, 1>{}, r + 1, cur, nid, more);
        }
        // every wave has finished reading this item's tiles: the ring is free
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // the next item's first V tile, unless the final interval (odd F) already sent it
        if (more && (steps & 1)) {
            const Item nx = make_item(nid);
            issue(nx.vview, lo_of(nx), vbuf(0));
        }
        bool write_out = true;
        if constexpr (SPLIT) {
            if (cur.part >= 0) write_out = merge_split(cur);
        }
        if (write_out) store_out(cur.id, cur.qi);
        if (write_out && a.lse != nullptr && hh == 0 && cur.qi < a.len) {
            // log-sum-exp of the scaled scores: m and l are in log2 units of c * s
            uint32_t r = cur.id % per_tile;
            const uint32_t hp = r % a.n_hpacks;
            r /= a.n_hpacks;
            const uint32_t kvh = r % a.Hkv;
            r /= a.Hkv;
            const uint32_t grp = r % a.groups;
            const uint32_t b = r / a.groups;
            const uint32_t h = kvh * a.G + hp * a.P + (uint32_t)wave % a.P;
            a.lse[((uint64_t)b * a.Hq + h) * a.N + (uint64_t)cur.qi * a.groups + grp] =
                (m_run + __builtin_amdgcn_logf(l_run)) * 0.6931471805599453f;
        }
        if (!more) break;
        cur = make_item(nid);
        ++round;
    }
}

// compute units of the current device (the persistent grid size)
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        __atomic_store_n(&cached[dev], c, __ATOMIC_RELAXED);
    }
    return c;
}

// Workgroups of the persistent grid: one per compute unit, unless the
// environment variable HD_SFA_PREFILL_WORKGROUPS holds a count from 1 to
// 65536 (a testing and tuning control).  Every work item is computed the same
// way whichever workgroup takes it, so the count never changes a result.
uint64_t persistent_workgroups() {
    uint64_t g = (uint64_t)device_cus();
    if (const char* e = std::getenv("HD_SFA_PREFILL_WORKGROUPS")) {
        char* end = nullptr;
        const long v = std::strtol(e, &end, 10);
        if (end != e && *end == '\0' && v >= 1 && v <= 65536) g = (uint64_t)v;
    }
    return g;
}

// Work items of a layer (see the kernel) and how many have two or more key
// tiles: the items a key-split launch takes in two halves.
struct ItemPlan {
    uint32_t n_qtiles = 0, per_tile = 0, BT = 0, P = 0;
    uint64_t items = 0, split_items = 0;
};
ItemPlan plan_items(int64_t B, int32_t n, int64_t L, int32_t Hq, int32_t Hkv, bool within) {
    ItemPlan p;
    const uint64_t len = within ? (uint64_t)L : (uint64_t)n * (uint64_t)L;
    const uint32_t G = (uint32_t)(Hq / Hkv);
    p.P = (G % 8 == 0) ? 8u : (G % 4 == 0) ? 4u : ((G % 2 == 0) ? 2u : 1u);
    p.BT = MQ * (NW / p.P);
    p.n_qtiles = (uint32_t)((len + p.BT - 1) / p.BT);
    p.per_tile = (uint32_t)B * (within ? (uint32_t)n : 1u) * (uint32_t)Hkv * (G / p.P);
    p.items = (uint64_t)p.n_qtiles * p.per_tile;
    // items are listed longest first; those of query tile qt end at key tile
    // ceil(min(len, (qt + 1) * BT) / BN)
    uint64_t qsplit = 0;
    for (uint64_t qt = 0; qt < p.n_qtiles; ++qt)
        if (std::min<uint64_t>(len, (qt + 1) * p.BT) > (uint64_t)BN) ++qsplit;
    p.split_items = qsplit * p.per_tile;
    return p;
}

// Workspace of a key-split launch: the (item, wave) counters, then two
// partial-state slots per (item, wave).
size_t split_counter_bytes(uint64_t split_items) {
    return ((size_t)split_items * NW * sizeof(uint32_t) + 255) & ~(size_t)255;
}
size_t split_workspace_bytes(uint64_t split_items, int32_t D) {
    if (split_items == 0) return 0;
    const size_t slot = (size_t)(D == 128 ? split_slot_floats<128>() : split_slot_floats<64>()) * sizeof(float);
    return split_counter_bytes(split_items) + (size_t)split_items * 2 * NW * slot;
}

hd_status launch_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         uint16_t* out, int64_t B, int32_t n, int64_t L, int32_t Hq,
                         int32_t Hkv, int32_t D, float scale, hipStream_t stream,
                         bool within, int64_t window, float* lse = nullptr,
                         void* split_ws = nullptr, size_t split_ws_bytes = 0) {
    // window: 0 = none (plain causal), else >= 1 rows of the view
    if (B < 0 || L < 0 || n < 1 || Hq < 1 || Hkv < 1 || window < 0) return HD_ERR_SHAPE;
    if (!scale_ok(scale)) return HD_ERR_SHAPE;
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
    a.lse = lse;
    a.Hq = (uint32_t)Hq;
    a.N = (uint32_t)N;

    const uint64_t items = (uint64_t)a.n_qtiles * a.B * a.groups * a.Hkv * a.n_hpacks;
    if (items > 0x7fffffffULL) return HD_ERR_UNSUPPORTED;
    a.n_items = (uint32_t)items;
    const uint64_t wgs = persistent_workgroups();
    // a window at least as long as the view masks nothing: the causal kernel
    const bool win = window > 0 && window < (int64_t)a.len;
    a.window = win ? (uint32_t)window : 0u;
    // key split: with a workspace, for a launch that gives no compute unit
    // more than one item (the causal items then differ in length up to the
    // number of key tiles and the longest sets the time)
    const ItemPlan plan = plan_items(B, n, L, Hq, Hkv, within);
    const bool split = split_ws != nullptr && !win && items <= wgs && plan.split_items > 0;
    a.n_split = split ? (uint32_t)plan.split_items : 0u;
    a.n_units = (uint32_t)items + a.n_split;
    a.cnt = nullptr;
    a.part = nullptr;
    if (split) {
        if (split_ws_bytes < split_workspace_bytes(plan.split_items, D) || !aligned16(split_ws))
            return HD_ERR_WORKSPACE;
        a.cnt = static_cast<uint32_t*>(split_ws);
        a.part = reinterpret_cast<float*>(static_cast<char*>(split_ws) + split_counter_bytes(plan.split_items));
    }
    const uint64_t blocks = a.n_units < wgs ? a.n_units : wgs;
    const int mode = a.c == 1.f ? kScaleLog2 : (scale == 1.f ? kScaleUnit : kScaleAny);
    auto pick = [&](auto d, auto w, auto sp) {
        constexpr int DD = decltype(d)::value;
        constexpr bool WW = decltype(w)::value;
        constexpr bool SS = decltype(sp)::value;
        return mode == kScaleLog2 ? sfa_prefill_kernel<DD, kScaleLog2, WW, SS>
             : mode == kScaleUnit ? sfa_prefill_kernel<DD, kScaleUnit, WW, SS>
                                  : sfa_prefill_kernel<DD, kScaleAny, WW, SS>;
    };
    using D128 = std::integral_constant<int, 128>;
    using D64 = std::integral_constant<int, 64>;
    using T1 = std::true_type;
    using T0 = std::false_type;
    auto kern = D == 128 ? (win ? pick(D128{}, T1{}, T0{}) : split ? pick(D128{}, T0{}, T1{}) : pick(D128{}, T0{}, T0{}))
                         : (win ? pick(D64{}, T1{}, T0{}) : split ? pick(D64{}, T0{}, T1{}) : pick(D64{}, T0{}, T0{}));
    kern<<<dim3((uint32_t)blocks), dim3(THREADS), 0, stream>>>(a);
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
                                 stream, /*within=*/true, /*window=*/0);
}

extern "C" hd_status sfa_mix_attn(const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, uint16_t* out, int64_t B,
                                  int32_t n, int64_t L, int32_t Hq, int32_t Hkv,
                                  int32_t D, float softmax_scale, hipStream_t stream) {
    return hdsfa::launch_prefill(q, k, v, out, B, n, L, Hq, Hkv, D, softmax_scale,
                                 stream, /*within=*/false, /*window=*/0);
}

extern "C" hd_status sfa_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  uint16_t* out, float* lse, int64_t B, int32_t n, int64_t L,
                                  int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                  int32_t mode, hipStream_t stream) {
    if (mode != 0 && mode != 1) return HD_ERR_SHAPE;
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return HD_ERR_SHAPE;
    return hdsfa::launch_prefill(q, k, v, out, B, n, L, Hq, Hkv, D, softmax_scale, stream,
                                 /*within=*/mode == 0, /*window=*/0, lse);
}

extern "C" size_t sfa_attn_split_workspace_size(int64_t B, int32_t n, int64_t L, int32_t Hq,
                                                int32_t Hkv, int32_t D, int32_t mode) {
    if (B < 1 || n < 1 || L < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return 0;
    if ((D != 64 && D != 128) || (mode != 0 && mode != 1)) return 0;
    const hdsfa::ItemPlan p = hdsfa::plan_items(B, n, L, Hq, Hkv, mode == 0);
    return hdsfa::split_workspace_bytes(p.split_items, D);
}

extern "C" hd_status sfa_attn_split(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    uint16_t* out, float* lse, int64_t B, int32_t n, int64_t L,
                                    int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                    int32_t mode, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    if (mode != 0 && mode != 1) return HD_ERR_SHAPE;
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return HD_ERR_SHAPE;
    if (workspace == nullptr && sfa_attn_split_workspace_size(B, n, L, Hq, Hkv, D, mode) > 0)
        return HD_ERR_WORKSPACE;
    return hdsfa::launch_prefill(q, k, v, out, B, n, L, Hq, Hkv, D, softmax_scale, stream,
                                 /*within=*/mode == 0, /*window=*/0, lse, workspace,
                                 workspace_bytes);
}

extern "C" hd_status sfa_mix_attn_window(const uint16_t* q, const uint16_t* k,
                                         const uint16_t* v, uint16_t* out, int64_t B,
                                         int32_t n, int64_t L, int32_t Hq, int32_t Hkv,
                                         int32_t D, float softmax_scale, int64_t window,
                                         hipStream_t stream) {
    if (window < 1) return HD_ERR_SHAPE;
    return hdsfa::launch_prefill(q, k, v, out, B, n, L, Hq, Hkv, D, softmax_scale,
                                 stream, /*within=*/false, window);
}


extern "C" hd_status sfa_attn_fwd_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         uint16_t* out, float* lse, int64_t B, int32_t n, int64_t L,
                                         int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                         int64_t window, hipStream_t stream) {
    if (window < 1) return HD_ERR_SHAPE;
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return HD_ERR_SHAPE;
    return hdsfa::launch_prefill(q, k, v, out, B, n, L, Hq, Hkv, D, softmax_scale, stream,
                                 /*within=*/false, window, lse);
}

// Chunkwise KDA forward for bfloat16 q, k, v on gfx950: a two-role pipeline
// inside one workgroup.
//
// One workgroup owns one (sequence, head, 64-wide slab of value columns) and
// walks the head's chunks of 64 tokens in order ("Kimi K3 - Lesson 3 of 14 -
// Sequence axis": sequential between chunks, parallel within; output =
// inter-chunk (Gamma . Q) S plus masked intra-chunk A V~; keys rescaled by
// 1/Gamma inside 16-token tiles, which the g_min = -5 floor keeps below
// e^80).  Everything a chunk needs that does not depend on the state is
// prepared one chunk ahead by four producer waves while four consumer waves
// run the state recurrence of the current chunk; the two sets hand over
// through a double-buffered LDS stage and meet at one workgroup barrier per
// chunk.  A SIMD holds one producer and one consumer wave, so the consumer's
// matrix-core work fills the producer's vector-ALU gaps and the other way
// round.
//
// Producer wave m, tile m (16 tokens; lane (g, r) holds token r and channels
// 16 blk + 4g + 0..3):
//   decays  b = within-tile inclusive cumsum of g (for bf16 gates one
//           matrix-core product per 16 channels with a constant triangle, g
//           read back transposed from LDS; for fp32 gates a DPP row scan),
//           f = e^b in [e^-80, 1], tile totals D_m (to LDS).
//   keys    K-hat_m: keys decayed to the end of tile m (B operands of the
//           later tiles' Gram blocks), to LDS; the last tile does its
//           diagonal Gram block meanwhile.  The four producers then meet at
//           an LDS counter (the consumers are not involved).
//   stage   Gamma.Q, Gamma.K (Gamma = decay from the chunk start) and K-bar
//           (keys decayed to the chunk end), and block row m of
//             A_qk (s <= t) and L = StrictLower(Diag(beta) A_kk),
//           A(t, s) = sum_c x_tc k_sc e^{b_tc - b_sc}.  The diagonal tile
//           pairs f-scaled rows with 1/f-scaled keys in two-term bfloat16
//           (the 1/f keys exceed fp16 range); a tile n = m - d pairs the
//           f-scaled rows times the whole tiles strictly between (D_{m-1},
//           D_{m-1} D_{m-2}) with K-hat_n, in fp16.
//   inverse (I + L_mm)^-1 by column-oriented forward substitution in fp32,
//           done at the top of the next chunk's iteration, beside its cumsum,
//           and counted for the consumers.
// Consumer wave 4 + w, value columns 16w..16w+15 of the slab, state slab
// S (dk x 16, fp32) in registers:
//   X = V - (Gamma.K) S,  U = (I + L)^-1 Diag(beta) X (blocked forward
//   substitution over the four tiles, once the chunk's four inverses are
//   counted), O = (Gamma.Q) S + A_qk U, S <- Diag(Gamma_C) S + K-bar^T U.
//
// Operand precision: fp16 single operands for (Gamma.Q) S, (Gamma.K) S, the
// off-diagonal Gram tiles and L U; fp16 two-term U (and right-hand sides of
// the diagonal inverses) against single fp16 A_qk, K-bar and inverses; fp32
// accumulation throughout.  fp16 needs the values, the state and the outputs
// to stay below 65504 in magnitude, which unit-scale values and L2-normalised
// queries and keys (as the method prescribes) satisfy.
#include <cstddef>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;             // tokens per chunk
constexpr int TILE = 16;          // tokens per tile
constexpr int NT = C / TILE;      // tiles per chunk
constexpr int NPROD = NT;         // producer waves: wave m prepares tile m
constexpr int NCONS = 4;          // consumer waves: 16 value columns each
constexpr int NTHREADS = 64 * (NPROD + NCONS);
constexpr int WV = 16 * NCONS;    // value columns per workgroup
constexpr int LDT = TILE;         // row stride (elements) of a stored 16x16 tile

// Element offset of the four-element group c (0..3) of row t of a stored
// 16x16 fp16 tile.  Rows are 32 bytes, so rows t and t + 8 fall in the same
// banks; rows 8..15 hold their groups in the order c ^ 2, so a half-wave
// writing rows 0..15 (groups 0,1 or 2,3) touches every bank once, and a
// transposed read (rows 4g + a, all four groups of each) still does.
__device__ __forceinline__ int tile_at(int t, int c) { return t * LDT + 4 * (c ^ ((t >> 2) & 2)); }
// The lane's address for a transposed read of such a tile (the offset
// h16::tr_offset gives for an unpermuted one, with the groups permuted).
__device__ __forceinline__ int tile_tr_offset(int lane) {
    return tile_at(4 * (lane >> 4) + ((lane & 15) >> 2), lane & 3);
}
constexpr float LOG2E = 1.4426950408889634f;

// Tiles (m, n) of the lower block triangle, n <= m, and of the strict one, n < m.
__host__ __device__ constexpr int lower_index(int m, int n) { return m * (m + 1) / 2 + n; }
__host__ __device__ constexpr int strict_index(int m, int n) { return m * (m - 1) / 2 + n; }
template <int M> struct TileIndex { static constexpr int value = M; };
constexpr int NLOWER = NT * (NT + 1) / 2;
constexpr int NSTRICT = NT * (NT - 1) / 2;

template <int DK>
struct alignas(16) PipeSmem {
    // Row strides (elements).  Token rows read four-at-a-time along channels
    // (Qt, Kt, Kh) are 16 bytes longer than a multiple of 256, so the 32 rows
    // x 8 bytes of a half-wave read fall in distinct banks; K-bar is read
    // transposed, four rows per 32-byte segment, and wants 32 bytes instead.
    static constexpr int LDK = DK + 8;
    static constexpr int LDKB = DK + 16;
    // What the consumers read for one chunk.
    struct alignas(16) Stage {
        _Float16 Qt[C * LDK];                   // Gamma . Q               [token][channel]
        _Float16 Kt[C * LDK];                   // Gamma . K               [token][channel]
        _Float16 Kb[C * LDKB];                  // K decayed to chunk end  [token][channel]
        _Float16 AqkT[NLOWER][TILE * LDT];      // tiles of A_qk, transposed: [s][t]
        _Float16 LT[NSTRICT][TILE * LDT];       // tiles of L, transposed
        _Float16 InvT[NT][TILE * LDT];          // (I + L_mm)^-1, transposed
        float GamC[DK];                         // total decay of the chunk
    };
    Stage stage[2];
    // Producer scratch.
    alignas(16) _Float16 Kh[NT - 1][TILE * LDK];   // keys of tiles 0..2 decayed to their tile end
    // total decay of each tile (read four channels at a time, one address per
    // lane group)
    alignas(16) float D[NT][DK];
    // beta of chunks c, c + 1, c + 2 (slot = chunk mod 3): written by a consumer
    // two iterations ahead, read by the producers one iteration ahead.
    alignas(16) float betas[3][C];
    // diagonal blocks of L (fp32): [m][col][row]; rows padded to 80 bytes so
    // that the 16 lanes of a quarter-wave reading 16 bytes of rows 0..15 hit
    // distinct banks
    alignas(16) float LdT[NT][TILE][TILE + 4];
    // bfloat16 gates of the next chunk for tiles 1..3 ([tile - 1][token][channel]),
    // loaded straight into LDS so that no registers hold them through the
    // staging pass (tile 0's producer, the lightest, keeps them in registers)
    alignas(16) uint16_t gnext[NT - 1][TILE * DK];
    unsigned arrivals;                          // producer meeting counter
    unsigned inv_posted;                        // diagonal inverses stored so far (all producers)
    unsigned failed;                            // some producer wait expired (read after the loop)
};

// Every array above is read with 8- or 16-byte LDS accesses.
static_assert(sizeof(PipeSmem<64>::Stage) % 16 == 0 && sizeof(PipeSmem<128>::Stage) % 16 == 0, "stage alignment");
static_assert(offsetof(PipeSmem<128>, betas) % 16 == 0 && offsetof(PipeSmem<128>, LdT) % 16 == 0 &&
              offsetof(PipeSmem<128>, D) % 16 == 0 && offsetof(PipeSmem<128>, Kh) % 16 == 0, "LDS alignment");
static_assert(offsetof(PipeSmem<64>, betas) % 16 == 0 && offsetof(PipeSmem<64>, LdT) % 16 == 0 &&
              offsetof(PipeSmem<64>, D) % 16 == 0 && offsetof(PipeSmem<64>, Kh) % 16 == 0, "LDS alignment");
static_assert(sizeof(PipeSmem<128>) <= 160 * 1024, "LDS budget of one workgroup");

// The q, k, g of one token row of one chunk, as raw storage bits.  A producer
// lane (g, r) holds token r of its tile, channels 16 blk + 4 g + (0..3).
template <int DK, typename GT>
struct RowIn {
    static constexpr int KT = DK / 16;
    Raw4<uint16_t> q[KT], k[KT];
    Raw4<GT> g[KT];
};

// The four producer waves meet here; LDS writes before it are visible to all
// four after it.  The wait is bounded (at most spin_limit sleeps); the result
// is false when it expired.  A launch in which any wait expired writes NaN
// over every output of the affected heads and their final states once the
// chunk loop is done, so an expired wait is never silent.
__device__ __forceinline__ bool producer_meet(unsigned *arrivals, unsigned target, int lane, unsigned spin_limit) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    bool ok = false;
    for (unsigned it = 0; it <= spin_limit; ++it) {
        const unsigned seen = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (seen >= target) { ok = true; break; }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    return ok;
}

// TR: slabs from nslab_v on are transition slabs.  Their dk "value" columns
// start from the identity with zero values and end as the columns of the
// chunk sequence's linear map on the state, M with S_out = M S_in + N (N the
// value slabs' final state from a zero start), written to M_out [b h][dk][dk];
// they write no output.
template <int DK, bool GBF, bool OBF, bool GL, bool TR = false>
__global__ void __launch_bounds__(NTHREADS, 1)
kda_chunk_pipe_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                      const uint16_t *__restrict__ v, const typename Store<GBF>::type *__restrict__ g,
                      const typename Store<GBF>::type *__restrict__ beta, const float *S0,
                      typename Store<OBF>::type *__restrict__ o, float *S_final,
                      const int *__restrict__ lengths, const float *__restrict__ A_log,
                      int B, int T, int H, int dv, int nslab, int nslab_v, float *M_out, unsigned spin_limit)
{
    typedef typename Store<GBF>::type GT;
    typedef typename Store<OBF>::type OT;
    typedef PipeSmem<DK> SM;
    typedef typename SM::Stage Stage;
    typedef Prec<true> BF;
    constexpr int KB = DK / 32;   // 32-channel blocks
    constexpr int KT = DK / 16;   // 16-channel tiles
    constexpr int LDK = SM::LDK, LDKB = SM::LDKB;

    __shared__ SM sm;

    const int lane = threadIdx.x & 63;
    // wave index, made explicitly uniform: every branch on it (and the
    // matrix-core instructions inside those branches, which ignore the exec
    // mask) stays scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool producer = wave < NPROD;
    const int r = lane & 15;     // row / column inside a 16x16 tile
    const int gq = lane >> 4;    // lane group: k-items, or output rows 4gq..4gq+3

    // Workgroup -> (b, h, slab).  Workgroups are dealt to the 8 XCDs round
    // robin; the slabs of one head go to the same XCD so they share its L2
    // for the q, k, g reads they have in common.
    const int BH = B * H;
    int bh, slab;
    if ((BH & 7) == 0) {
        const int rest = blockIdx.x >> 3;
        slab = rest % nslab;
        bh = (rest / nslab) * 8 + (blockIdx.x & 7);
    } else {
        bh = blockIdx.x / nslab;
        slab = blockIdx.x % nslab;
    }
    const int b = bh / H, h = bh % H;
    const int nchunks = (T + C - 1) / C;
    // tokens from `len` on are identity tokens (no decay, no write)
    const int len = lengths ? max(0, min(lengths[b], T)) : T;

    // Between two workgroup barriers the producers prepare chunk c + 1 into
    // stage (c + 1) & 1 while the consumers run chunk c from stage c & 1.  Each
    // role runs its own loop; both pass the same nchunks + 2 barriers.
    if (producer) {
        const int m = wave;   // tile
        const float gate_scale = GL ? __expf(A_log[h]) : 1.f;   // exp(A_h), gate logits only
        RowIn<DK, GT> in;     // inputs of the next chunk to prepare
        // Loads of chunk c: g as soon as the scan has consumed the previous
        // chunk's, q and k once the staging has consumed theirs.  Every load
        // is issued unconditionally (a token past the end reads the last
        // token; its g is zeroed when used, and its zero beta keeps it from
        // writing), so the loads in flight are always the same ones and
        // waiting for g never waits for the younger q and k loads.
        auto token_row = [&](int c, int r) -> size_t {
            const int t = min(c * C + TILE * m + r, T - 1);
            return ((size_t)b * T + t) * H + h;
        };
        auto load_g = [&](int c, int r, int gq) {
            const GT *gb = g + token_row(c, r) * DK + 4 * gq;
#pragma unroll
            for (int blk = 0; blk < KT; ++blk) in.g[blk].load(gb + 16 * blk);
        };
        // q and k come through buffer loads based at the chunk's first token row
        // (the launcher keeps a chunk's byte span below 2^31).  A plain load
        // from these read-only arrays is ordered with nothing else in its basic
        // block, and the compiler issued the next chunk's after the inverse
        // below, a whole phase late; a buffer load stays ahead of the LDS
        // writes that follow it.
        // channel blocks blk0 .. blk1 - 1 of this lane's row
        auto load_qk_blocks = [&](int c, int r, int gq, int blk0, int blk1) {
            const size_t row0 = (((size_t)b * T + (size_t)c * C) * H + h) * DK;
            const auto qr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(q + row0), (short)0, (int)0xFFFFFFFF, 0x00020000);
            const auto kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(k + row0), (short)0, (int)0xFFFFFFFF, 0x00020000);
            const int t = min(TILE * m + r, T - 1 - c * C);   // as token_row
            const uint32_t off = (uint32_t)t * (uint32_t)(H * DK * 2) + 8u * (uint32_t)gq;
#pragma unroll
            for (int blk = blk0; blk < blk1; ++blk) {
                if constexpr (!TR) {   // transition passes form no output: no queries
                    const u32x2 qv = __builtin_amdgcn_raw_buffer_load_b64(qr, off + 32u * blk, 0, 0);
                    in.q[blk].a = make_uint2(qv.x, qv.y);
                }
                const u32x2 kv = __builtin_amdgcn_raw_buffer_load_b64(kr, off + 32u * blk, 0, 0);
                in.k[blk].a = make_uint2(kv.x, kv.y);
            }
        };
        auto load_qk = [&](int c, int r, int gq) { load_qk_blocks(c, r, gq, 0, KT); };

        if (threadIdx.x == 0) {
            sm.arrivals = 0;
            sm.inv_posted = 0;
            sm.failed = 0;
        }
        if (nchunks == 0) {
            lds_barrier();
            lds_barrier();
            return;
        }
        // bfloat16 gates (not logits) of tiles 1..3 come through sm.gnext:
        // DK / 32 LDS-direct loads of 1 KB per chunk (a token row is DK / 8
        // lanes of 16 bytes), issued from inline assembly so the compiler does
        // not make every later LDS read wait for them; the loop top waits for
        // them by count (only the 2 KT q and k loads are younger)
        constexpr bool GDMA = GBF && !GL;
        constexpr int GROW_LANES = DK / 8;          // lanes per token row
        constexpr int GROWS = 64 / GROW_LANES;      // token rows per load
        static_assert(TILE % GROWS == 0, "whole loads per tile");
        auto dma_g = [&](int c, int tm) {
            const unsigned base = (unsigned)(size_t)&sm.gnext[tm - 1][0];
#pragma unroll
            for (int j = 0; j < TILE / GROWS; ++j) {
                const GT *src = g + token_row(c, GROWS * j + lane / GROW_LANES) * DK + 8 * (lane % GROW_LANES);
                const unsigned dst = __builtin_amdgcn_readfirstlane(base + 1024u * j);
                asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
            }
        };
        unsigned meetings = 0;   // producer meetings so far (uniform)
        bool all_met = true;     // every meeting completed within its bound
        // One loop instance per tile: the tile's work, and which of its values
        // stay live through the loop, are fixed at compile time.
        auto tile_loop = [&](auto tile) __attribute__((always_inline)) {
        constexpr int M = decltype(tile)::value;
        constexpr bool GLDS = GDMA && M >= 1;   // this tile's gates come through LDS
        if constexpr (GLDS) dma_g(0, M);
        else load_g(0, r, gq);
        load_qk(0, r, gq);   // after the gates: the loop top's count relies on the order
        // this tile's L block starts as zero (the first, unused inverse is then I)
        for (int i = lane; i < TILE * (TILE + 4); i += 64) (&sm.LdT[M][0][0])[i] = 0.f;
        lds_barrier();
        // (I + L_mm)^-1 of chunk c, lane column r, stored transposed into the
        // chunk's stage and counted in inv_posted.  It runs at the top of the
        // next iteration (the L block stays in LdT until that iteration's block
        // row), beside the next chunk's cumsum rather than after this chunk's
        // block row; the consumers wait for the count before their solve.  At c
        // = -1 it inverts the zeroed LdT into stage 1, which chunk 1 rewrites
        // before any consumer reads it.
        auto invert_chunk = [&](int c) __attribute__((always_inline)) {
            int r = lane & 15, gq = lane >> 4;
            asm volatile("" : "+v"(r), "+v"(gq));
            // column r of L_mm, and X = e_r; `one` is opaque so the 16 selects
            // are not hoisted out of the chunk loop
            float Lc[TILE];
#pragma unroll
            for (int i4 = 0; i4 < TILE / 4; ++i4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&sm.LdT[M][r][4 * i4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) Lc[4 * i4 + i] = x[i];
            }
            float one = 1.f;
            asm volatile("" : "+v"(one));
            float X[TILE];
#pragma unroll
            for (int i = 0; i < TILE; ++i) X[i] = (i == r) ? one : 0.f;
            unit_lower_inverse_steps<0>(X, Lc);
            // lane group gq stores rows 4gq..4gq+3 of column r (row r of the
            // transpose), chosen by masks from the two bits of gq: a chain of
            // equality tests on gq compiles to nested branches, and a select
            // between array elements to a select of addresses (the array then
            // lives in scratch memory)
            f32x4 part;
            const unsigned m1 = (gq & 1) ? ~0u : 0u, m2 = (gq & 2) ? ~0u : 0u;
            auto pick = [](float a, float b, unsigned m) {
                return __uint_as_float(__float_as_uint(a) ^ ((__float_as_uint(a) ^ __float_as_uint(b)) & m));
            };
#pragma unroll
            for (int i = 0; i < 4; ++i) part[i] = pick(pick(X[i], X[4 + i], m1), pick(X[8 + i], X[12 + i], m1), m2);
            *reinterpret_cast<f16x4 *>(&sm.stage[c & 1].InvT[M][tile_at(r, gq)]) = h16::pack4(part);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            if (lane == 0) __hip_atomic_fetch_add(&sm.inv_posted, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        for (int cn = 0; cn < nchunks; ++cn) {
            {
                Stage &st = sm.stage[cn & 1];
                // Lane coordinates made opaque here, so that no address derived from
                // them is computed once before the loop and held in a register (or
                // spilled) through it: every iteration recomputes what it uses.
                int r = lane & 15, gq = lane >> 4;
                asm volatile("" : "+v"(r), "+v"(gq));
                const bool live = cn * C + TILE * m + r < len;   // else: identity token
                const int cnext = min(cn + 1, nchunks - 1);    // the last chunk reloads itself

                // ---------------------------------------------- decays within tile m
                // b = inclusive cumsum of g over the tile's 16 tokens, per channel
                float f[KT][4];   // f = e^b in [e^-80, 1] (1/f, up to e^80, is recomputed where used)
                if constexpr (GLDS) {
                    // the gates' LDS-direct loads are complete once at most the 2 KT
                    // q and k loads issued after them (KT k loads in a transition
                    // pass) are outstanding
                    constexpr int YOUNGER = TR ? KT : 2 * KT;
                    static_assert(YOUNGER < 64, "vmcnt field");
                    __builtin_amdgcn_s_waitcnt(0x0F70 | (YOUNGER & 15) | ((YOUNGER >> 4) << 14));
                    // Tri(s, t) = [s <= t], with the rows of tokens past the end zeroed:
                    // identity tokens (g = 0) drop out of every sum
                    i16x4 tri;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        tri[i] = (4 * gq + i <= r && cn * C + TILE * M + 4 * gq + i < len) ? (short)0x3F80 : (short)0;   // bf16 1.0
                    const int tro = h16::tr_offset(lane, DK);
                    const _Float16 *gsrc = reinterpret_cast<const _Float16 *>(&sm.gnext[M - 1][0]);
#pragma unroll
                    for (int blk = 0; blk < KT; ++blk) {
                        // channels as rows, tokens 4 gq + i as k-items
                        const i16x4 gt = __builtin_bit_cast(i16x4, h16::tr4(gsrc + 16 * blk + tro));
                        const f32x4 bsum = BF::mma16(gt, tri, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i) f[blk][i] = fast_exp2(bsum[i] * LOG2E);
                    }
                } else if constexpr (GBF && !GL) {
                    // as a matrix-core product: b^T = g^T Tri, Tri(s, t) = [s <= t].
                    // g goes through this tile's rows of the Qt staging area (rewritten
                    // below) as KT stored 16x16 tiles, read back transposed: channels
                    // as rows, tokens as k-items.
                    static_assert(KT * TILE * LDT <= TILE * LDK, "g staging fits the tile's Qt rows");
                    uint16_t *gs = reinterpret_cast<uint16_t *>(&st.Qt[TILE * m * LDK]);
#pragma unroll
                    for (int blk = 0; blk < KT; ++blk)
                        *reinterpret_cast<uint2 *>(&gs[TILE * LDT * blk + tile_at(r, gq)]) =
                            live ? in.g[blk].a : make_uint2(0, 0);
                    lds_wave_sync();
                    i16x4 tri;
#pragma unroll
                    for (int i = 0; i < 4; ++i) tri[i] = (4 * gq + i <= r) ? (short)0x3F80 : (short)0;   // bf16 1.0
                    const int tro = tile_tr_offset(lane);
#pragma unroll
                    for (int blk = 0; blk < KT; ++blk) {
                        const i16x4 gt = __builtin_bit_cast(
                            i16x4, h16::tr4(reinterpret_cast<const _Float16 *>(&gs[TILE * LDT * blk + tro])));
                        const f32x4 bsum = BF::mma16(gt, tri, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i) f[blk][i] = fast_exp2(bsum[i] * LOG2E);
                    }
                } else {
                    // float32 gates, or gates computed here from logits: a DPP scan
                    // across the 16 lanes of each row
#pragma unroll
                    for (int blk = 0; blk < KT; ++blk) {
                        float gl[4];
                        in.g[blk].to_f32(gl);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if constexpr (GL) gl[i] = gate_from_logit(gl[i], gate_scale);
                            f[blk][i] = fast_exp2(row_inclusive_scan(live ? gl[i] * LOG2E : 0.f));
                        }
                    }
                }
                invert_chunk(cn - 1);
                if (r == TILE - 1) {
#pragma unroll
                    for (int blk = 0; blk < KT; ++blk)
                        *reinterpret_cast<f32x4 *>(&sm.D[m][16 * blk + 4 * gq]) =
                            f32x4{f[blk][0], f[blk][1], f[blk][2], f[blk][3]};
                }
                if constexpr (!GLDS) load_g(cnext, r, gq);
                lds_wave_sync();

                // diagonal Gram tile, block (m, m): f-scaled rows against 1/f-scaled
                // keys of the same tile, two-term bfloat16.  k-items of block pair p:
                // channels 32p + 4gq + (0..3) and 32p + 16 + 4gq + (0..3).
                f32x4 gq_d = {0.f, 0.f, 0.f, 0.f}, gk_d = {0.f, 0.f, 0.f, 0.f};
                auto diagonal = [&](const float (&qf)[8], const float (&kf)[8], const float (&ki)[8]) {
                    if constexpr (!TR) {
                        BF::frag8 aqh, aql, bih, bil;
                        BF::split8(qf, aqh, aql);
                        BF::split8(ki, bih, bil);
                        const BF::frag8 akh = BF::pack8(kf);
                        gq_d = BF::mma32(aqh, bih, gq_d);
                        gq_d = BF::mma32(aqh, bil, gq_d);
                        gq_d = BF::mma32(aql, bih, gq_d);
                        gk_d = BF::mma32(akh, bih, gk_d);
                    } else {   // no output: only the key-key block
                        BF::frag8 bih, bil;
                        BF::split8(ki, bih, bil);
                        gk_d = BF::mma32(BF::pack8(kf), bih, gk_d);
                    }
                };

                if constexpr (M < NT - 1) {
                    // keys decayed to the end of tile m: B operands of the later tiles' Gram blocks
#pragma unroll
                    for (int blk = 0; blk < KT; ++blk) {
                        const int ch = 16 * blk + 4 * gq;
                        const f32x4 dm = *reinterpret_cast<const f32x4 *>(&sm.D[m][ch]);
                        float kv[4];
                        in.k[blk].to_f32(kv);
                        f32x4 kh;
#pragma unroll
                        for (int i = 0; i < 4; ++i) kh[i] = kv[i] * fast_rcp(f[blk][i]) * dm[i];
                        *reinterpret_cast<f16x4 *>(&sm.Kh[m][r * LDK + ch]) = h16::pack4(kh);
                    }
                } else {
                    // the last tile has no keys to hand on: it does its diagonal tile
                    // here, while the others write theirs
#pragma unroll
                    for (int p = 0; p < KB; ++p) {
                        float qf[8], kf[8], ki[8];
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            float qv[4], kv[4];
                            if constexpr (!TR) in.q[2 * p + hh].to_f32(qv);
                            else qv[0] = qv[1] = qv[2] = qv[3] = 0.f;
                            in.k[2 * p + hh].to_f32(kv);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                qf[4 * hh + i] = qv[i] * f[2 * p + hh][i];
                                kf[4 * hh + i] = kv[i] * f[2 * p + hh][i];
                                ki[4 * hh + i] = kv[i] * fast_rcp(f[2 * p + hh][i]);
                            }
                        }
                        diagonal(qf, kf, ki);
                    }
                }
                // the next chunk's gates (tiles 1..3): after every use of this chunk's
                // gates and of the q, k loaded before them
                if constexpr (GLDS) dma_g(cnext, M);
                meetings += 1;
                all_met = producer_meet(&sm.arrivals, NPROD * meetings, lane, spin_limit) && all_met;

                // ---------------------------------------------- staged operands and block row m of the Gram
                // Instantiated once per tile: which Gram tiles exist and the
                // whole-tile decays between tiles are then fixed at compile time,
                // with no per-tile branches (and no register copies merging them).
                auto block_row = [&](auto tile) __attribute__((always_inline)) {
                    constexpr int M = decltype(tile)::value;
                    f32x4 gq_o[NT - 1], gk_o[NT - 1];
#pragma unroll
                    for (int d = 0; d < NT - 1; ++d) {
                        gq_o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
                        gk_o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                    for (int p = 0; p < KB; ++p) {
                        float qf[8], kf[8], ki[8], v2[8], v3[8];
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int blk = 2 * p + hh;
                            const int ch = 16 * blk + 4 * gq;
                            // the four tiles' totals of these 4 channels (each read is
                            // one address per lane group, broadcast to its 16 lanes)
                            f32x4 Dt[NT];
#pragma unroll
                            for (int t = 0; t < NT; ++t) Dt[t] = *reinterpret_cast<const f32x4 *>(&sm.D[t][ch]);
                            // whole-tile decay before tile M, from its start to the chunk
                            // end, and across the tiles strictly between M and M - 2, M - 3
                            f32x4 before = {1.f, 1.f, 1.f, 1.f}, dma = Dt[M], w2 = before, w3 = before;
#pragma unroll
                            for (int t = 0; t < M; ++t) before = t ? before * Dt[t] : Dt[t];
#pragma unroll
                            for (int t = M + 1; t < NT; ++t) dma = dma * Dt[t];
                            if constexpr (M >= 2) w2 = Dt[M - 1];
                            if constexpr (M >= 3) w3 = Dt[M - 1] * Dt[M - 2];
                            if constexpr (M == 0)
                                if (r == 0) *reinterpret_cast<f32x4 *>(&st.GamC[ch]) = dma;
                            float qv[4], kv[4];
                            if constexpr (!TR) in.q[blk].to_f32(qv);
                            else qv[0] = qv[1] = qv[2] = qv[3] = 0.f;
                            in.k[blk].to_f32(kv);
                            f32x4 qt, kt, kb;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float fq = qv[i] * f[blk][i], fk = kv[i] * f[blk][i];
                                const float ik = kv[i] * fast_rcp(f[blk][i]);   // 1/f-scaled key, <= e^80 |k|
                                qf[4 * hh + i] = fq;
                                kf[4 * hh + i] = fk;
                                ki[4 * hh + i] = ik;
                                v2[4 * hh + i] = w2[i];
                                v3[4 * hh + i] = w3[i];
                                qt[i] = M ? fq * before[i] : fq;
                                kt[i] = M ? fk * before[i] : fk;
                                kb[i] = ik * dma[i];   // decayed to the chunk end, <= |k|
                            }
                            const int row = (TILE * M + r) * LDK + ch;
                            if constexpr (!TR) *reinterpret_cast<f16x4 *>(&st.Qt[row]) = h16::pack4(qt);
                            *reinterpret_cast<f16x4 *>(&st.Kt[row]) = h16::pack4(kt);
                            *reinterpret_cast<f16x4 *>(&st.Kb[(TILE * M + r) * LDKB + ch]) = h16::pack4(kb);
                        }

                        if constexpr (M < NT - 1) diagonal(qf, kf, ki);
                        // tiles n = M - d to the left: fp16, B = K-hat of tile n
                        const int kh_off = r * LDK + 32 * p + 4 * gq;
                        if constexpr (M >= 1) {
                            const f16x8 bk = h16::lds4x2(&sm.Kh[M - 1][kh_off], &sm.Kh[M - 1][kh_off + 16]);
                            if constexpr (!TR) gq_o[0] = h16::mma32(h16::pack8(qf), bk, gq_o[0]);
                            gk_o[0] = h16::mma32(h16::pack8(kf), bk, gk_o[0]);
                        }
                        if constexpr (M >= 2) {
                            const f16x8 bk = h16::lds4x2(&sm.Kh[M - 2][kh_off], &sm.Kh[M - 2][kh_off + 16]);
                            float a[8], e[8];
#pragma unroll
                            for (int i = 0; i < 8; ++i) { a[i] = qf[i] * v2[i]; e[i] = kf[i] * v2[i]; }
                            if constexpr (!TR) gq_o[1] = h16::mma32(h16::pack8(a), bk, gq_o[1]);
                            gk_o[1] = h16::mma32(h16::pack8(e), bk, gk_o[1]);
                        }
                        if constexpr (M >= 3) {
                            const f16x8 bk = h16::lds4x2(&sm.Kh[M - 3][kh_off], &sm.Kh[M - 3][kh_off + 16]);
                            float a[8], e[8];
#pragma unroll
                            for (int i = 0; i < 8; ++i) { a[i] = qf[i] * v3[i]; e[i] = kf[i] * v3[i]; }
                            if constexpr (!TR) gq_o[2] = h16::mma32(h16::pack8(a), bk, gq_o[2]);
                            gk_o[2] = h16::mma32(h16::pack8(e), bk, gk_o[2]);
                        }
                        // this block pair's q and k are consumed: fetch the next chunk's
                        load_qk_blocks(cnext, r, gq, 2 * p, 2 * p + 2);
                    }

                    lds_wave_sync();

                    // ------------------------------------------ Gram results of block row M
                    const f32x4 bet = *reinterpret_cast<const f32x4 *>(&sm.betas[cn % 3][TILE * M + 4 * gq]);
                    {
                        f32x4 aq, ak;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int row = 4 * gq + i;   // row t inside the tile; the column s is r
                            aq[i] = (r > row) ? 0.f : gq_d[i];             // keep s <= t
                            ak[i] = (r >= row) ? 0.f : gk_d[i] * bet[i];   // keep s <  t
                        }
                        if constexpr (!TR) *reinterpret_cast<f16x4 *>(&st.AqkT[lower_index(M, M)][tile_at(r, gq)]) = h16::pack4(aq);
                        *reinterpret_cast<f32x4 *>(&sm.LdT[M][r][4 * gq]) = ak;
                    }
#pragma unroll
                    for (int d = 1; d <= M; ++d) {
                        const int n = M - d;
                        if constexpr (!TR)
                            *reinterpret_cast<f16x4 *>(&st.AqkT[lower_index(M, n)][tile_at(r, gq)]) =
                                h16::pack4(gq_o[d - 1]);
                        *reinterpret_cast<f16x4 *>(&st.LT[strict_index(M, n)][tile_at(r, gq)]) =
                            h16::pack4(gk_o[d - 1] * bet);
                    }
                    lds_wave_sync();
                };
                block_row(TileIndex<M>{});
                // the machine scheduler may not move the next chunk's q, k loads
                // (issued in the block row) down past the inverse either
                __builtin_amdgcn_sched_barrier(0);
            }
            lds_barrier();
        }
        invert_chunk(nchunks - 1);
        };
        static_assert(NT == 4, "one loop instance per tile");
        switch (m) {
        case 0: tile_loop(TileIndex<0>{}); break;
        case 1: tile_loop(TileIndex<1>{}); break;
        case 2: tile_loop(TileIndex<2>{}); break;
        default: tile_loop(TileIndex<3>{}); break;
        }
        if (!all_met && lane == 0) sm.failed = 1u;
        lds_barrier();   // the consumers' last chunk
    } else {
        const int w = wave - NPROD;                 // column group
        const bool trans = TR && slab >= nslab_v;   // a transition slab (uniform)
        const int col0 = (trans ? slab - nslab_v : slab) * WV + 16 * w;   // first column of this consumer
        const int lds = trans ? DK : dv;            // row stride of this slab's state matrix
        float *const S_out = trans ? M_out : S_final;
        const size_t s_base = (size_t)bh * DK * lds + col0 + r;
        const size_t Hdv = (size_t)H * dv;
        const uint32_t lane_v = (uint32_t)(4 * gq * H * dv + r);   // rows 4gq + i, column r

        f32x4 S[KT];           // rows 16kt + 4gq + i, column r
        uint16_t vin[NT][4];   // V rows 16mm + 4gq + i, column r, of the chunk being computed
        uint16_t vnx[NT][4];   // the same for the next chunk
        // V and o of this consumer's columns are addressed through buffer
        // resources based at the chunk's first row: the row's byte offset inside
        // the chunk is a scalar (soffset), the lane's column and row group a fixed
        // voffset, so no vector instruction computes an address (the launcher
        // keeps these offsets below 2^31).
        const uint16_t *v_head = v + ((size_t)b * T * H + h) * dv + col0;
        OT *o_head = (o && !trans) ? o + ((size_t)b * T * H + h) * dv + col0 : nullptr;
        const uint32_t v_stride = (uint32_t)Hdv * 2u, o_stride = (uint32_t)Hdv * (uint32_t)sizeof(OT);
        auto rsrc = [](const void *base) {
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)0xFFFFFFFF, 0x00020000);
        };
        // V of chunk c.  A token past the end reads the last token instead (its
        // beta is zero, so its value never enters U).
        auto load_v = [&](int c, uint16_t (&dst)[NT][4]) {
            if (trans) {   // zero values
#pragma unroll
                for (int mm = 0; mm < NT; ++mm)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[mm][i] = 0;
                return;
            }
            const auto vr = rsrc(v_head + (size_t)c * C * Hdv);
            if ((c + 1) * C <= T) {
#pragma unroll
                for (int mm = 0; mm < NT; ++mm)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[mm][i] = __builtin_amdgcn_raw_buffer_load_b16(vr, lane_v * 2u, (uint32_t)(TILE * mm + i) * v_stride, 0);
            } else {
#pragma unroll
                for (int mm = 0; mm < NT; ++mm)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = min(TILE * mm + 4 * gq + i, T - 1 - c * C);
                        dst[mm][i] = __builtin_amdgcn_raw_buffer_load_b16(vr, (uint32_t)t * v_stride + 2u * r, 0u, 0);
                    }
            }
        };

        // beta: consumer 0 keeps the slots two chunks ahead, one token per lane
        auto load_beta = [&](int c) -> GT {
            const int t = c * C + lane;
            return t < len ? beta[((size_t)b * T + t) * H + h] : GT(0);
        };
        GT bnext = GT(0);   // beta of chunk c + 2, written into its slot in iteration c
        if (w == 0) {
            sm.betas[0][lane] = nchunks > 0 ? to_f32(load_beta(0)) : 0.f;
            sm.betas[1][lane] = nchunks > 1 ? to_f32(load_beta(1)) : 0.f;
            if (nchunks > 2) bnext = load_beta(2);
        }

#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[kt][i] = trans ? (16 * kt + 4 * gq + i == col0 + r ? 1.f : 0.f)
                                 : S0 ? S0[s_base + (size_t)(16 * kt + 4 * gq + i) * dv] : 0.f;
        if (nchunks > 0) load_v(0, vin);
        lds_barrier();

        // One chunk of the recurrence.  The next chunk's V is requested first;
        // LDS operands are read ahead of the products that use them: the
        // state-independent tiles first, each row tile's scaled queries and
        // keys while the previous row tile's products run, K-bar during the
        // output products.  Scheduling fences keep the compiler from sinking
        // the reads back next to their uses.
        auto chunk_step = [&](int c) __attribute__((always_inline)) {
            // this chunk's V (requested a chunk ago) and the previous chunk's
            // output stores are complete; the compiler's wait tracking learns it here
            __builtin_amdgcn_s_waitcnt(0x0F70);
            if (c + 1 < nchunks) load_v(c + 1, vnx);
            const Stage &st = sm.stage[c & 1];
            const int tro = tile_tr_offset(lane);

            // ---- operands that do not depend on the state
            f16x4 lt[NSTRICT];
#pragma unroll
            for (int i = 0; i < NSTRICT; ++i) lt[i] = h16::tr4(&st.LT[i][tro]);
            f32x4 bts[NT];
            row_gather16(sm.betas[c % 3][TILE * (r >> 2) + 4 * gq + (r & 3)], bts);
            // scaled queries and keys of row tile mm: k-items channels 32j + 4gq + i and 32j + 16 + 4gq + i
            f16x8 aq[2][KB], ak[2][KB];
            auto load_rows = [&](int mm, f16x8 (&q8)[KB], f16x8 (&k8)[KB]) {
                const int row = (TILE * mm + r) * LDK;
#pragma unroll
                for (int j = 0; j < KB; ++j) {
                    const int ch = row + 32 * j + 4 * gq;
                    if constexpr (!TR) q8[j] = h16::lds4x2(&st.Qt[ch], &st.Qt[ch + 16]);   // (no output: no Gamma.Q)
                    k8[j] = h16::lds4x2(&st.Kt[ch], &st.Kt[ch + 16]);
                }
            };
            load_rows(0, aq[0], ak[0]);

            // state slab as fp16 operands: k-items = channels 32j + 4gq + i and 32j + 16 + 4gq + i
            f16x8 Sh[KB];
#pragma unroll
            for (int j = 0; j < KB; ++j) Sh[j] = h16::pack8(S[2 * j], S[2 * j + 1]);

            // ---- (Gamma.Q) S, computed transposed (the state slab as A operand,
            // the scaled queries as B): lane (g, r) then holds output columns
            // 4g..4g+3 of token r, four consecutive values for one wide store;
            // and Y = beta (V - (Gamma.K) S) in the state's own layout
            f32x4 accQ[NT], Y[NT];
#pragma unroll
            for (int mm = 0; mm < NT; ++mm) {
                if (mm + 1 < NT) load_rows(mm + 1, aq[(mm + 1) & 1], ak[(mm + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                f32x4 aQ = {0.f, 0.f, 0.f, 0.f}, aK = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < KB; ++j) {
                    if constexpr (!TR) aQ = h16::mma32(Sh[j], aq[mm & 1][j], aQ);
                    aK = h16::mma32(ak[mm & 1][j], Sh[j], aK);
                }
                accQ[mm] = aQ;
#pragma unroll
                for (int i = 0; i < 4; ++i) Y[mm][i] = bts[mm][i] * (to_f32(vin[mm][i]) - aK[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (w == 0 && c + 2 < nchunks) sm.betas[(c + 2) % 3][lane] = to_f32(bnext);

            // ---- A_qk tiles, read while the solve runs
            f16x4 aqk[NLOWER];
#pragma unroll
            for (int i = 0; i < NLOWER; ++i)
                if constexpr (!TR) aqk[i] = h16::tr4(&st.AqkT[i][tro]);

            // ---- the diagonal inverses of this chunk: the producers store them at
            // the start of this period (four per chunk, counted from the first
            // period on); a bounded wait, failing loudly like theirs
            {
                bool ok = false;
                const unsigned want = 4u * (unsigned)(c + 2);
                for (unsigned it = 0; it <= spin_limit; ++it) {
                    const unsigned seen = __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(&sm.inv_posted, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
                    if (seen >= want) { ok = true; break; }
                    __builtin_amdgcn_s_sleep(1);
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                if (!ok && lane == 0) sm.failed = 1u;
            }
            f16x4 inv[NT];
#pragma unroll
            for (int mm = 0; mm < NT; ++mm) inv[mm] = h16::tr4(&st.InvT[mm][tro]);
            // ---- U = (I + L)^-1 Diag(beta) X, one tile at a time
            f16x4 Uh[NT], Ul[NT];
#pragma unroll
            for (int mm = 0; mm < NT; ++mm) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int n = 0; n < mm; ++n) acc = h16::mma16(lt[strict_index(mm, n)], Uh[n], acc);
                f16x4 rh, rl;
                h16::split4(Y[mm] - acc, rh, rl);
                f32x4 uu = h16::mma16(inv[mm], rh, f32x4{0.f, 0.f, 0.f, 0.f});
                uu = h16::mma16(inv[mm], rl, uu);
                h16::split4(uu, Uh[mm], Ul[mm]);
            }
            __builtin_amdgcn_sched_barrier(0);

            // ---- K-bar^T operands of the first half of the state row tiles, read during the output products
            const int tk = h16::tr_offset(lane, LDKB);
            auto load_kb = [&](int kt, f16x8 (&k8)[2]) {
#pragma unroll
                for (int j2 = 0; j2 < 2; ++j2) {
                    const _Float16 *base = &st.Kb[(32 * j2) * LDKB + 16 * kt + tk];
                    k8[j2] = __builtin_shufflevector(h16::tr4(base), h16::tr4(base + 16 * LDKB), 0, 1, 2, 3, 4, 5, 6, 7);
                }
            };
            f16x8 kb[KT][2];
#pragma unroll
            for (int kt = 0; kt < KT / 2; ++kt) load_kb(kt, kb[kt]);
            // total decay of the chunk for rows 16kt + 4gq + (0..3), four row
            // tiles per LDS read (one value per lane, shared across the row)
            static_assert(KT % 4 == 0, "row tiles of the state come in fours");
            f32x4 gam[KT / 4][4];
#pragma unroll
            for (int q4 = 0; q4 < KT / 4; ++q4) row_gather16(st.GamC[16 * (4 * q4 + (r >> 2)) + 4 * gq + (r & 3)], gam[q4]);
            __builtin_amdgcn_sched_barrier(0);

            // ---- O^T = ((Gamma.Q) S)^T + U^T A_qk^T (U as the A operand, the A_qk
            // tiles as B): lane (g, r) holds four consecutive columns of token r,
            // one wide store per row tile
            if (!TR && o_head) {
                const auto orr = rsrc(o_head + (size_t)c * C * Hdv);
                const uint32_t o_lane = (uint32_t)r * o_stride + (uint32_t)(4 * gq) * (uint32_t)sizeof(OT);
#pragma unroll
                for (int mm = 0; mm < NT; ++mm) {
                    f32x4 acc = accQ[mm];
#pragma unroll
                    for (int n = 0; n <= mm; ++n) {
                        acc = h16::mma16(Uh[n], aqk[lower_index(mm, n)], acc);
                        acc = h16::mma16(Ul[n], aqk[lower_index(mm, n)], acc);
                    }
                    if (c * C + TILE * mm + r < T) {
                        if constexpr (OBF)
                            __builtin_amdgcn_raw_buffer_store_b64(
                                u32x2{(uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16),
                                      (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16)},
                                orr, o_lane, (uint32_t)(TILE * mm) * o_stride, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), orr, o_lane,
                                                                   (uint32_t)(TILE * mm) * o_stride, 0);
                    }
                }
            }
#pragma unroll
            for (int kt = KT / 2; kt < KT; ++kt) load_kb(kt, kb[kt]);
            __builtin_amdgcn_sched_barrier(0);

            // ---- S <- Diag(Gamma_C) S + K-bar^T U, U's two fp16 terms as 8-item B operands
            // (k-items: the tokens of tiles 2 j2 and 2 j2 + 1)
            f16x8 Ubh[2], Ubl[2];
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2) {
                Ubh[j2] = __builtin_shufflevector(Uh[2 * j2], Uh[2 * j2 + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                Ubl[j2] = __builtin_shufflevector(Ul[2 * j2], Ul[2 * j2 + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                f32x4 acc = S[kt] * gam[kt / 4][kt % 4];
#pragma unroll
                for (int j2 = 0; j2 < 2; ++j2) {
                    acc = h16::mma32(kb[kt][j2], Ubh[j2], acc);
                    acc = h16::mma32(kb[kt][j2], Ubl[j2], acc);
                }
                S[kt] = acc;
            }
            if (w == 0 && c + 3 < nchunks) bnext = load_beta(c + 3);
        };
        for (int c = -1; c < nchunks; ++c) {
            if (c >= 0) {
                chunk_step(c);
#pragma unroll
                for (int mm = 0; mm < NT; ++mm)
#pragma unroll
                    for (int i = 0; i < 4; ++i) vin[mm][i] = vnx[mm][i];
            }
            lds_barrier();
        }
        if (__builtin_amdgcn_readfirstlane(sm.failed) != 0u) {
            // a producer wait expired somewhere in the sequence: its operands may
            // have been built from unfinished data, so nothing this workgroup
            // wrote stands; every output of its columns and its state become NaN
            const float nan = __builtin_nanf("");
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) S[kt] = f32x4{nan, nan, nan, nan};
            if (o_head)
                for (int t = 4 * gq; t < T; t += 16)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (t + i < T) o[(((size_t)b * T + t + i) * H + h) * dv + col0 + r] = from_f32<OT>(nan);
        }
        if (S_out) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S_out[s_base + (size_t)(16 * kt + 4 * gq + i) * lds] = S[kt][i];
        }
    }
}

template <int DK, bool GBF, bool OBF, bool GL>
hipError_t launch(const ChunkFwdArgs &a, hipStream_t stream)
{
    typedef typename Store<GBF>::type GT;
    typedef typename Store<OBF>::type OT;
    const int nslab = a.dv / WV;
    const unsigned grid = (unsigned)(a.B * a.H * nslab);
    kda_chunk_pipe_kernel<DK, GBF, OBF, GL><<<grid, NTHREADS, 0, stream>>>(
        (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, (const GT *)a.g,
        (const GT *)a.beta, a.S0, (OT *)a.o, a.S_final, a.lengths, a.A_log, a.B, a.T, a.H, a.dv, nslab, nslab,
        nullptr, spin_limit());
    return hipGetLastError();
}

// The value slabs' final states from a zero start (a.S_final) and the chunk
// sequence's linear map (M_out), no outputs; bf16 or fp32 gates, or gate
// logits with a.A_log; no per-sequence lengths.
template <int DK, bool GBF, bool GL>
hipError_t launch_trans(const ChunkFwdArgs &a, float *M_out, hipStream_t stream)
{
    typedef typename Store<GBF>::type GT;
    const int nslab_v = a.dv / WV, nslab = nslab_v + DK / WV;
    const unsigned grid = (unsigned)(a.B * a.H * nslab);
    kda_chunk_pipe_kernel<DK, GBF, false, GL, true><<<grid, NTHREADS, 0, stream>>>(
        (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, (const GT *)a.g,
        (const GT *)a.beta, nullptr, nullptr, a.S_final, nullptr, a.A_log, a.B, a.T, a.H, a.dv, nslab, nslab_v,
        M_out, spin_limit());
    return hipGetLastError();
}

template <int DK>
hipError_t dispatch_trans(const ChunkFwdArgs &a, float *M_out, hipStream_t s)
{
    if (a.A_log)
        return a.gate_bf16 ? launch_trans<DK, true, true>(a, M_out, s) : launch_trans<DK, false, true>(a, M_out, s);
    return a.gate_bf16 ? launch_trans<DK, true, false>(a, M_out, s) : launch_trans<DK, false, false>(a, M_out, s);
}

template <int DK, bool GL>
hipError_t dispatch_gate(const ChunkFwdArgs &a, hipStream_t s)
{
    if (a.gate_bf16) return a.out_bf16 ? launch<DK, true, true, GL>(a, s) : launch<DK, true, false, GL>(a, s);
    return a.out_bf16 ? launch<DK, false, true, GL>(a, s) : launch<DK, false, false, GL>(a, s);
}

template <int DK>
hipError_t dispatch(const ChunkFwdArgs &a, hipStream_t s)
{
    return a.A_log ? dispatch_gate<DK, true>(a, s) : dispatch_gate<DK, false>(a, s);
}

}  // namespace

hipError_t launch_chunk_fwd_bf16_trans(const ChunkFwdArgs &a, float *M_out, hipStream_t stream)
{
    (void)hipGetLastError();
    if ((uint64_t)C * a.H * a.dv * 4 + (uint64_t)a.H * a.dv * 4 >= ((uint64_t)1 << 31)) return hipErrorInvalidValue;
    if ((uint64_t)C * a.H * a.dk * 2 + (uint64_t)a.H * a.dk * 2 >= ((uint64_t)1 << 31)) return hipErrorInvalidValue;
    if (a.lengths || !M_out) return hipErrorInvalidValue;
    return a.dk == 64 ? dispatch_trans<64>(a, M_out, stream) : dispatch_trans<128>(a, M_out, stream);
}

hipError_t launch_chunk_fwd_bf16(const ChunkFwdArgs &a, hipStream_t stream)
{
    (void)hipGetLastError();   // report only this launch's own failure
    // buffer offsets inside one chunk (64 rows of H * dv values for V and o, of
    // H * dk for q and k) stay 32-bit
    if ((uint64_t)C * a.H * a.dv * 4 + (uint64_t)a.H * a.dv * 4 >= ((uint64_t)1 << 31)) return hipErrorInvalidValue;
    if ((uint64_t)C * a.H * a.dk * 2 + (uint64_t)a.H * a.dk * 2 >= ((uint64_t)1 << 31)) return hipErrorInvalidValue;
    if (a.dk == 64) return dispatch<64>(a, stream);
    return dispatch<128>(a, stream);
}

}  // namespace kda

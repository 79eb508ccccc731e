// Chunkwise KDA forward for bfloat16 q, k, v on gfx950: prep and state
// workgroups in pairs, joined through a ring of chunk slots held in L2.
//
// The chunkwise form ("Kimi K3 - Lesson 3 of 14 - Sequence axis": sequential
// between chunks, parallel within; output = inter-chunk (Gamma . Q) S plus
// masked intra-chunk A V~; keys rescaled by 1/Gamma inside 16-token tiles,
// which the g_min = -5 floor keeps below e^80) splits into work that does not
// depend on the state (decays, scaled operands, Gram tiles, the diagonal
// inverses: everything a chunk needs before it meets S) and the state
// recurrence itself.  Here each head gets one prep workgroup, which computes
// the state-independent part of every chunk exactly once, and 1..4 state
// workgroups (128 value columns each), which run the recurrence.  The prep
// workgroup writes each chunk's operands into a slot of a three-slot ring in
// the caller's workspace; the state workgroups copy the slot into LDS with
// LDS-direct loads one chunk ahead and hand the slot back.  The ring is small
// (3 x 63 KB per head) and lives in the L2 of the XCD that runs the head.
//
// Synchronisation.  All workgroups of a head run on one XCD (workgroup i is
// dispatched to XCD i mod 8; each workgroup checks this at run time), so the
// XCD's L2 is the point where the two sides meet: slot data and flags are
// written with ordinary stores (complete once s_waitcnt vmcnt(0) returns) and
// read with loads that bypass the CU's L1 (device scope, sc1).  Flags are
// 64-bit: the launch's epoch in the high half (a per-process counter, started
// at a random value and advanced per launch) and the chunk number + 1 in the
// low half; a wait accepts only the exact value it expects, so flags of other
// launches and uninitialised memory never satisfy it and the workspace needs
// no clearing.  Every wait is bounded by `spin_limit` sleeps;
// when a bound expires the waiting side marks the call failed (low half all
// ones), never overwrites a slot the other side may still read, and the
// state side sets its state to NaN, which carries into every output from then
// on and the final state: a failed call is loud, and every wave still runs to
// its end.  The launch is cooperative, so all
// workgroups of the grid are resident together.
//
// Arithmetic and operand formats are those of kda_chunk_pipe.hip (the same
// producer and consumer steps, in the same order), so the two kernels give
// the same results.
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cstddef>

#include "kda_chunk_tiles.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

using namespace chunk;

constexpr int NWAVE = 8;
constexpr int NTHREADS = 64 * NWAVE;
constexpr int NTEAM = 2;              // prep teams: team t prepares chunks t, t + 2, ...
constexpr int NPROD = NT;             // waves per team: one per tile
constexpr int SCOLS = 16 * NWAVE;     // value columns of one state workgroup
constexpr int RING = 3;               // slots per head
constexpr int MAXSTATE = 4;           // state workgroups per head (dv <= 512)
constexpr size_t FLAG_BYTES = 512;    // per head: ready line, consumed line, info line
constexpr uint32_t FAILED = 0xFFFFFFFFu;

// What the state workgroups read for one chunk; the same bytes in the ring
// slot (global memory) and in an LDS stage.
template <int DK>
struct alignas(16) Slot {
    // Row strides (elements).  Token rows read four-at-a-time along channels
    // (Qt, Kt) are 16 bytes longer than a multiple of 256, so the 32 rows x 8
    // bytes of a half-wave read fall in distinct banks; K-bar is read
    // transposed, four rows per 32-byte segment, and wants 32 bytes instead.
    static constexpr int LDK = DK + 8;
    static constexpr int LDKB = DK + 16;
    _Float16 Qt[C * LDK];                   // Gamma . Q               [token][channel]
    _Float16 Kt[C * LDK];                   // Gamma . K               [token][channel]
    _Float16 Kb[C * LDKB];                  // K decayed to chunk end  [token][channel]
    _Float16 AqkT[NLOWER][TILE * LDT];      // tiles of A_qk, transposed: [s][t]
    _Float16 LT[NSTRICT][TILE * LDT];       // tiles of L, transposed
    _Float16 InvT[NT][TILE * LDT];          // (I + L_mm)^-1, transposed
    float GamC[DK];                         // total decay of the chunk
    float beta[C];                          // beta of the chunk's tokens (0 past the end)
};
static_assert(sizeof(Slot<128>) % 16 == 0 && sizeof(Slot<64>) % 16 == 0, "slot copies move 16-byte units");

// Scratch of one prep team (LDS).
template <int DK>
struct alignas(16) TeamSmem {
    static constexpr int LDK = DK + 8;
    static constexpr int LDD = DK + 16;     // rows 64 bytes longer than DK floats (bank spread of the gathers)
    _Float16 gst[NT][DK / 16][TILE * LDT];  // gates of each tile, staged for the transposed read
    _Float16 Kh[NT - 1][TILE * LDK];        // keys of tiles 0..2 decayed to their tile end
    float D[NT][LDD];                       // total decay of each tile
    float LdT[NT][TILE][TILE + 4];          // diagonal blocks of L (fp32): [m][col][row], 80-byte rows
    float betas[C];                         // beta of the chunk being prepared
    unsigned arrivals;                      // team meeting counter
    unsigned go;                            // leader's verdict on the slot wait (1: proceed)
};

template <int DK>
struct alignas(16) StateSmem {
    Slot<DK> stage[2];
    unsigned failed;                        // set by any wave whose wait expired
};

template <int DK>
union alignas(16) PsSmem {
    StateSmem<DK> state;
    TeamSmem<DK> team[NTEAM];
};
static_assert(sizeof(PsSmem<128>) <= 160 * 1024, "LDS budget of one workgroup");
static_assert(offsetof(Slot<128>, AqkT) % 16 == 0 && offsetof(Slot<128>, GamC) % 16 == 0 &&
              offsetof(Slot<128>, Kb) % 16 == 0 && offsetof(Slot<128>, beta) % 16 == 0, "slot alignment");
static_assert(offsetof(TeamSmem<128>, Kh) % 16 == 0 && offsetof(TeamSmem<128>, D) % 16 == 0 &&
              offsetof(TeamSmem<128>, LdT) % 16 == 0 && offsetof(TeamSmem<128>, betas) % 16 == 0, "team alignment");

// ------------------------------------------------------------ cross-workgroup flags

__device__ __forceinline__ uint64_t tag(uint32_t epoch, uint32_t v) { return ((uint64_t)epoch << 32) | v; }

// Device-scope (sc1) accesses: the load misses the CU's L1 and reads the
// XCD's L2, the store writes through to it.
__device__ __forceinline__ uint64_t poll64(const uint64_t *p) {
    const uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void post64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every vector-memory access of this wave issued so far has completed (for
// stores: reached the L2).
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Waits until *p holds `want` or `fail`, starting from an already polled
// value; at most `limit` sleeps.  Returns the last value seen; `ok` is
// cleared on expiry.  Exact matches only: memory that never held a flag of
// this launch (an uninitialised workspace, flags of earlier launches) never
// satisfies a wait.
__device__ __forceinline__ uint64_t wait_flag(const uint64_t *p, uint64_t want, uint64_t fail, uint64_t seen,
                                              unsigned limit, bool &ok) {
    for (unsigned it = 0; seen != want && seen != fail; ++it) {
        if (it >= limit) { ok = false; break; }
        __builtin_amdgcn_s_sleep(1);
        seen = poll64(p);
    }
    return seen;
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds + 16 i.  Issued from inline assembly so the compiler does not make
// every later LDS read wait for it; the caller waits (wait_vm) before reading
// the destination.  Device scope, so the bytes come from the L2.
__device__ __forceinline__ void lds_dma16(const void *src, unsigned lds) {
    asm volatile("global_load_lds_dwordx4 %0, off sc1" ::"v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint32_t xcc_id() {
    return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11));   // HW_REG_XCC_ID, bits 0..15
}

struct PsArgs {
    const uint16_t *q, *k, *v;
    const void *g, *beta;
    const float *S0;
    void *o;
    float *S_final;
    const float *A_log;
    unsigned char *ws;       // flags, then slots
    size_t slot_off;         // byte offset of the slots in ws
    int B, T, H, dv, nstate, h_begin, G;
    uint32_t epoch;
    unsigned spin_limit;
};

template <int DK, bool GBF, bool OBF, bool GL>
__global__ void __launch_bounds__(NTHREADS, 1) kda_chunk_ps_kernel(PsArgs a)
{
    typedef typename Store<GBF>::type GT;
    typedef typename Store<OBF>::type OT;
    typedef Slot<DK> SL;
    typedef Prec<true> BF;
    constexpr int KB = DK / 32;   // 32-channel blocks
    constexpr int KT = DK / 16;   // 16-channel tiles
    constexpr int LDK = SL::LDK, LDKB = SL::LDKB;
    constexpr int SLOT_U4 = (int)(sizeof(SL) / 16);
    constexpr int NCOPY = (SLOT_U4 + NTHREADS - 1) / NTHREADS;

    __shared__ PsSmem<DK> sm;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;     // row / column inside a 16x16 tile
    const int gq = lane >> 4;    // lane group: k-items, or output rows 4gq..4gq+3

    // Workgroup -> (head, role).  Workgroup i runs on XCD i mod 8; the 1 + nstate
    // workgroups of a head are i = 8 (u P + role) + x, all on XCD x.
    const int P = 1 + a.nstate;
    const int x = blockIdx.x & 7, s = blockIdx.x >> 3;
    const int u = s / P, role = s - u * P;
    const int hl = u * 8 + x;   // head within this launch's group
    if (hl >= a.G) return;
    const int bh = a.h_begin + hl;
    const int b = bh / a.H, h = bh % a.H;
    const int T = a.T, H = a.H, dv = a.dv;
    const int nchunks = (T + C - 1) / C;
    const uint32_t epoch = a.epoch;
    const unsigned limit = a.spin_limit;

    uint64_t *flags = reinterpret_cast<uint64_t *>(a.ws + (size_t)hl * FLAG_BYTES);
    uint64_t *ready = flags;              // [RING], written by the prep workgroup
    uint64_t *consumed = flags + 16;      // [RING][MAXSTATE], written by the state workgroups
    uint64_t *info = flags + 32;          // [0]: the prep workgroup's XCD, tagged with the epoch
    SL *slots = reinterpret_cast<SL *>(a.ws + a.slot_off) + (size_t)hl * RING;

    if (role == 0) {
        // ====================================================== prep workgroup
        const GT *g = static_cast<const GT *>(a.g);
        const GT *beta = static_cast<const GT *>(a.beta);
        const int team = wave / NPROD;
        const int wt = wave % NPROD;
        // the second team's waves take the tiles in rotated order, so each SIMD
        // (wave i runs on SIMD i mod 4) holds a light and a heavy tile
        const int m = team == 0 ? wt : (wt + 2) % NT;
        const bool leader = wt == 0;
        TeamSmem<DK> &ts = sm.team[team];
        const float gate_scale = GL ? __expf(a.A_log[h]) : 1.f;

        if (threadIdx.x == 0) post64(info, tag(epoch, xcc_id()));
        if (lane == 0 && wt == 0) ts.arrivals = 0;
        __syncthreads();

        RowIn<DK, GT> in;    // inputs of the team's next chunk
        GT bnext = GT(0);    // its beta (tile-0 wave: lane = token)
        auto token_row = [&](int c, int rr) -> size_t {
            const int t = min(c * C + TILE * m + rr, T - 1);
            return ((size_t)b * T + t) * H + h;
        };
        auto load_g = [&](int c) {
            const GT *gb = g + token_row(c, r) * DK + 4 * gq;
#pragma unroll
            for (int blk = 0; blk < KT; ++blk) in.g[blk].load(gb + 16 * blk);
        };
        auto load_qk = [&](int c) {
            const size_t off = token_row(c, r) * DK + 4 * gq;
#pragma unroll
            for (int blk = 0; blk < KT; ++blk) {
                in.q[blk].load(a.q + off + 16 * blk);
                in.k[blk].load(a.k + off + 16 * blk);
            }
        };
        auto load_beta = [&](int c) -> GT {
            const int t = c * C + lane;
            return t < T ? beta[((size_t)b * T + t) * H + h] : GT(0);
        };

        unsigned meetings = 0;
        bool ok = true;
        if (team < nchunks) {
            load_g(team);
            load_qk(team);
            if (m == 0) bnext = load_beta(team);
        }
        for (int cn = team; cn < nchunks && ok; cn += NTEAM) {
            const int slot = cn % RING;
            SL *st = slots + slot;
            int r = lane & 15, gq = lane >> 4;
            asm volatile("" : "+v"(r), "+v"(gq));
            const bool live = cn * C + TILE * m + r < T;   // else: identity token
            const int cnext = cn + NTEAM < nchunks ? cn + NTEAM : cn;
            // the leader's poll of the slot's consumers, issued early
            uint64_t seen[MAXSTATE] = {0, 0, 0, 0};
            const uint64_t want = tag(epoch, (uint32_t)(cn - RING + 1));
            if (leader && cn >= RING)
                for (int j = 0; j < a.nstate; ++j) seen[j] = poll64(&consumed[slot * MAXSTATE + j]);

            // ---------------------------------------------- decays within tile m
            float f[KT][4];   // f = e^b in [e^-80, 1]
            if constexpr (GBF && !GL) {
                uint16_t *gs = reinterpret_cast<uint16_t *>(&ts.gst[m][0][0]);
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
            if (r == TILE - 1) {
#pragma unroll
                for (int blk = 0; blk < KT; ++blk)
                    *reinterpret_cast<f32x4 *>(&ts.D[m][16 * blk + 4 * gq]) =
                        f32x4{f[blk][0], f[blk][1], f[blk][2], f[blk][3]};
            }
            float bcur = 0.f;
            if (m == 0) {
                bcur = to_f32(bnext);
                ts.betas[lane] = bcur;
                bnext = load_beta(cnext);
            }
            load_g(cnext);
            lds_wave_sync();

            // diagonal Gram tile, block (m, m): f-scaled rows against 1/f-scaled
            // keys of the same tile, two-term bfloat16.
            f32x4 gq_d = {0.f, 0.f, 0.f, 0.f}, gk_d = {0.f, 0.f, 0.f, 0.f};
            auto diagonal = [&](const float (&qf)[8], const float (&kf)[8], const float (&ki)[8]) {
                BF::frag8 aqh, aql, bih, bil;
                BF::split8(qf, aqh, aql);
                BF::split8(ki, bih, bil);
                const BF::frag8 akh = BF::pack8(kf);
                gq_d = BF::mma32(aqh, bih, gq_d);
                gq_d = BF::mma32(aqh, bil, gq_d);
                gq_d = BF::mma32(aql, bih, gq_d);
                gk_d = BF::mma32(akh, bih, gk_d);
            };

            if (m < NT - 1) {
#pragma unroll
                for (int blk = 0; blk < KT; ++blk) {
                    const int ch = 16 * blk + 4 * gq;
                    const f32x4 dm = *reinterpret_cast<const f32x4 *>(&ts.D[m][ch]);
                    float kv[4];
                    in.k[blk].to_f32(kv);
                    f32x4 kh;
#pragma unroll
                    for (int i = 0; i < 4; ++i) kh[i] = kv[i] * fast_rcp(f[blk][i]) * dm[i];
                    *reinterpret_cast<f16x4 *>(&ts.Kh[m][r * LDK + ch]) = h16::pack4(kh);
                }
            } else {
#pragma unroll
                for (int p = 0; p < KB; ++p) {
                    float qf[8], kf[8], ki[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        float qv[4], kv[4];
                        in.q[2 * p + hh].to_f32(qv);
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

            // the slot is free once every state workgroup has copied the chunk
            // that used it last
            if (leader) {
                bool free_ok = true;
                if (cn >= RING)
                    for (int j = 0; j < a.nstate; ++j)
                        wait_flag(&consumed[slot * MAXSTATE + j], want, tag(epoch, FAILED), seen[j], limit, free_ok);
                if (lane == 0) ts.go = free_ok ? 1u : 0u;
            }
            meetings += 1;
            ok = lds_meet(&ts.arrivals, NPROD * meetings, lane, limit);
            ok = ok && ts.go != 0;
            if (!ok) break;

            // ---------------------------------------------- staged operands and block row m of the Gram
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
                        f32x4 Dt[NT];
                        row_gather16(ts.D[r >> 2][ch + (r & 3)], Dt);
                        f32x4 before = {1.f, 1.f, 1.f, 1.f}, dma = Dt[M], w2 = before, w3 = before;
#pragma unroll
                        for (int t = 0; t < M; ++t) before = t ? before * Dt[t] : Dt[t];
#pragma unroll
                        for (int t = M + 1; t < NT; ++t) dma = dma * Dt[t];
                        if constexpr (M >= 2) w2 = Dt[M - 1];
                        if constexpr (M >= 3) w3 = Dt[M - 1] * Dt[M - 2];
                        if constexpr (M == 0)
                            if (r == 0) *reinterpret_cast<f32x4 *>(&st->GamC[ch]) = dma;
                        float qv[4], kv[4];
                        in.q[blk].to_f32(qv);
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
                        *reinterpret_cast<f16x4 *>(&st->Qt[row]) = h16::pack4(qt);
                        *reinterpret_cast<f16x4 *>(&st->Kt[row]) = h16::pack4(kt);
                        *reinterpret_cast<f16x4 *>(&st->Kb[(TILE * M + r) * LDKB + ch]) = h16::pack4(kb);
                    }

                    if constexpr (M < NT - 1) diagonal(qf, kf, ki);
                    const int kh_off = r * LDK + 32 * p + 4 * gq;
                    if constexpr (M >= 1) {
                        const f16x8 bk = h16::lds4x2(&ts.Kh[M - 1][kh_off], &ts.Kh[M - 1][kh_off + 16]);
                        gq_o[0] = h16::mma32(h16::pack8(qf), bk, gq_o[0]);
                        gk_o[0] = h16::mma32(h16::pack8(kf), bk, gk_o[0]);
                    }
                    if constexpr (M >= 2) {
                        const f16x8 bk = h16::lds4x2(&ts.Kh[M - 2][kh_off], &ts.Kh[M - 2][kh_off + 16]);
                        float aa[8], e[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) { aa[i] = qf[i] * v2[i]; e[i] = kf[i] * v2[i]; }
                        gq_o[1] = h16::mma32(h16::pack8(aa), bk, gq_o[1]);
                        gk_o[1] = h16::mma32(h16::pack8(e), bk, gk_o[1]);
                    }
                    if constexpr (M >= 3) {
                        const f16x8 bk = h16::lds4x2(&ts.Kh[M - 3][kh_off], &ts.Kh[M - 3][kh_off + 16]);
                        float aa[8], e[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) { aa[i] = qf[i] * v3[i]; e[i] = kf[i] * v3[i]; }
                        gq_o[2] = h16::mma32(h16::pack8(aa), bk, gq_o[2]);
                        gk_o[2] = h16::mma32(h16::pack8(e), bk, gk_o[2]);
                    }
                }

                // q and k of chunk cn are consumed: fetch the team's next chunk's
                load_qk(cnext);

                // ------------------------------------------ Gram results of block row M
                const f32x4 bet = *reinterpret_cast<const f32x4 *>(&ts.betas[TILE * M + 4 * gq]);
                {
                    f32x4 aq, ak;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 4 * gq + i;   // row t inside the tile; the column s is r
                        aq[i] = (r > row) ? 0.f : gq_d[i];             // keep s <= t
                        ak[i] = (r >= row) ? 0.f : gk_d[i] * bet[i];   // keep s <  t
                    }
                    *reinterpret_cast<f16x4 *>(&st->AqkT[lower_index(M, M)][tile_at(r, gq)]) = h16::pack4(aq);
                    *reinterpret_cast<f32x4 *>(&ts.LdT[M][r][4 * gq]) = ak;
                }
#pragma unroll
                for (int d = 1; d <= M; ++d) {
                    const int n = M - d;
                    *reinterpret_cast<f16x4 *>(&st->AqkT[lower_index(M, n)][tile_at(r, gq)]) =
                        h16::pack4(gq_o[d - 1]);
                    *reinterpret_cast<f16x4 *>(&st->LT[strict_index(M, n)][tile_at(r, gq)]) =
                        h16::pack4(gk_o[d - 1] * bet);
                }
                lds_wave_sync();
            };
            static_assert(NT == 4, "one block_row instance per tile");
            switch (m) {
            case 0: block_row(TileIndex<0>{}); break;
            case 1: block_row(TileIndex<1>{}); break;
            case 2: block_row(TileIndex<2>{}); break;
            default: block_row(TileIndex<3>{}); break;
            }
            if (m == 0) st->beta[lane] = bcur;

            // ------------------------------------------ (I + L_mm)^-1, lane column r
            {
                float Lc[TILE];
#pragma unroll
                for (int i4 = 0; i4 < TILE / 4; ++i4) {
                    const f32x4 xx = *reinterpret_cast<const f32x4 *>(&ts.LdT[m][r][4 * i4]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Lc[4 * i4 + i] = xx[i];
                }
                float one = 1.f;
                asm volatile("" : "+v"(one));
                float X[TILE];
#pragma unroll
                for (int i = 0; i < TILE; ++i) X[i] = (i == r) ? one : 0.f;
                unit_lower_inverse_steps<0>(X, Lc);
                f32x4 part;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    part[i] = gq == 0 ? X[i] : gq == 1 ? X[4 + i] : gq == 2 ? X[8 + i] : X[12 + i];
                *reinterpret_cast<f16x4 *>(&st->InvT[m][tile_at(r, gq)]) = h16::pack4(part);
            }

            // every store of this chunk has reached the L2 in all four waves:
            // publish the slot
            wait_vm();
            meetings += 1;
            ok = lds_meet(&ts.arrivals, NPROD * meetings, lane, limit);
            if (ok && leader && lane == 0) post64(&ready[slot], tag(epoch, (uint32_t)(cn + 1)));
        }
        if (!ok && leader && lane == 0) {
            // a wait expired: the state side stops waiting and writes NaN
            for (int sl = 0; sl < RING; ++sl) post64(&ready[sl], tag(epoch, FAILED));
        }
        return;
    }

    // ========================================================== state workgroup
    const int jst = role - 1;
    const int w = wave;
    const int col0 = SCOLS * jst + 16 * w;        // first value column of this wave
    const bool active = col0 < dv;                // uniform
    typedef StateSmem<DK> SS;
    SS &ss = sm.state;
    const size_t s_base = (size_t)bh * DK * dv + col0 + r;
    const size_t Hdv = (size_t)H * dv;
    const uint32_t lane_v = (uint32_t)(4 * gq * H * dv + r);   // rows 4gq + i, column r
    OT *o = static_cast<OT *>(a.o);

    if (threadIdx.x == 0) ss.failed = 0u;
    lds_barrier();

    f32x4 S[KT];           // rows 16kt + 4gq + i, column r
    uint16_t vin[NT][4];   // V rows 16mm + 4gq + i, column r, of the chunk being computed
    uint16_t vnx[NT][4];   // the same for the next chunk
    // V and o of this wave's column group are addressed through buffer
    // resources based at the chunk's first row: the row's byte offset inside
    // the chunk is a scalar (soffset), the lane's column and row group a fixed
    // voffset, so no vector instruction computes an address.
    const uint16_t *v_head = a.v + ((size_t)b * T * H + h) * dv + col0;
    OT *o_head = o ? o + ((size_t)b * T * H + h) * dv + col0 : nullptr;
    const uint32_t v_stride = (uint32_t)Hdv * 2u, o_stride = (uint32_t)Hdv * (uint32_t)sizeof(OT);
    auto rsrc = [](const void *base) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)0xFFFFFFFF, 0x00020000);
    };
    auto load_v = [&](int c, uint16_t (&dst)[NT][4]) {
        const auto vr = rsrc(v_head + (size_t)c * C * Hdv);
        if ((c + 1) * C <= T) {
#pragma unroll
            for (int mm = 0; mm < NT; ++mm)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[mm][i] = __builtin_amdgcn_raw_buffer_load_b16(vr, lane_v * 2u, (uint32_t)(TILE * mm + i) * v_stride, 0);
        } else {
            // a token past the end reads the last token instead (its beta is zero)
#pragma unroll
            for (int mm = 0; mm < NT; ++mm)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = min(TILE * mm + 4 * gq + i, T - 1 - c * C);
                    dst[mm][i] = __builtin_amdgcn_raw_buffer_load_b16(vr, (uint32_t)t * v_stride + 2u * r, 0u, 0);
                }
        }
    };
    // copy of chunk c's slot into stage c & 1, this thread's share
    auto copy_slot = [&](int c) {
        const uint4 *src = reinterpret_cast<const uint4 *>(slots + c % RING);
        const unsigned base = (unsigned)(size_t)&ss.stage[c & 1];
#pragma unroll
        for (int u2 = 0; u2 < NCOPY; ++u2) {
            const int idx = u2 * NTHREADS + (int)threadIdx.x;
            const unsigned dst = __builtin_amdgcn_readfirstlane(base + (unsigned)(u2 * NTHREADS + 64 * wave) * 16u);
            if (idx < SLOT_U4) lds_dma16(src + idx, dst);
        }
    };
    // this wave's verdict on chunk c's slot: ready, or the wait expired or the
    // prep side failed
    auto slot_ok = [&](int c, uint64_t first) -> bool {
        bool ok = true;
        const uint64_t seen =
            wait_flag(&ready[c % RING], tag(epoch, (uint32_t)(c + 1)), tag(epoch, FAILED), first, limit, ok);
        return ok && (uint32_t)seen != FAILED;
    };

#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[kt][i] = (active && a.S0) ? a.S0[s_base + (size_t)(16 * kt + 4 * gq + i) * dv] : 0.f;

    bool failed = false;
    uint64_t pend = 0;   // polled value of the next chunk's ready flag
    if (nchunks > 0) {
        bool okc = slot_ok(0, poll64(&ready[0]));
        // every workgroup of the head must sit on the XCD whose L2 carries the ring
        if (okc && poll64(info) != tag(epoch, xcc_id())) okc = false;
        if (okc) copy_slot(0);
        else if (lane == 0) ss.failed = 1u;
        if (active) load_v(0, vin);
        if (nchunks > 1) pend = poll64(&ready[1 % RING]);
    }
    wait_vm();
    lds_barrier();
    failed = ss.failed != 0u;
    if (nchunks > 0 && w == 0 && lane == 0)
        post64(&consumed[0 * MAXSTATE + jst], tag(epoch, failed ? FAILED : 1u));

    for (int c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) {
            if (!failed) {
                const bool okc = slot_ok(c + 1, pend);
                if (okc) copy_slot(c + 1);
                else if (lane == 0) ss.failed = 1u;
                if (c + 2 < nchunks) pend = poll64(&ready[(c + 2) % RING]);
            }
            if (active) load_v(c + 1, vnx);
        }
        if (active) {
            const SL &st = ss.stage[c & 1];
            if (failed) {
                // this chunk's stage was not filled: the state turns NaN, and with it
                // every output from here on and the final state
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) S[kt] = f32x4{1.f, 1.f, 1.f, 1.f} * __builtin_nanf("");
            }

            // state slab as fp16 B operands: k-items = channels 32j + 4gq + i and 32j + 16 + 4gq + i
            f16x8 Sh[KB];
#pragma unroll
            for (int j = 0; j < KB; ++j) Sh[j] = h16::pack8(S[2 * j], S[2 * j + 1]);

            // (Gamma.Q) S and X = V - (Gamma.K) S, scaled by beta
            f32x4 accQ[NT], Y[NT], bts[NT];
            row_gather16(st.beta[TILE * (r >> 2) + 4 * gq + (r & 3)], bts);
#pragma unroll
            for (int mm = 0; mm < NT; ++mm) {
                f32x4 aQ = {0.f, 0.f, 0.f, 0.f}, aK = {0.f, 0.f, 0.f, 0.f};
                const int row = (TILE * mm + r) * LDK;
#pragma unroll
                for (int j = 0; j < KB; ++j) {
                    const int ch = row + 32 * j + 4 * gq;
                    aQ = h16::mma32(h16::lds4x2(&st.Qt[ch], &st.Qt[ch + 16]), Sh[j], aQ);
                    aK = h16::mma32(h16::lds4x2(&st.Kt[ch], &st.Kt[ch + 16]), Sh[j], aK);
                }
                accQ[mm] = aQ;
#pragma unroll
                for (int i = 0; i < 4; ++i) Y[mm][i] = bts[mm][i] * (to_f32(vin[mm][i]) - aK[i]);
            }

            // U = (I + L)^-1 Diag(beta) X, one tile at a time
            const int tro = tile_tr_offset(lane);
            f16x4 Uh[NT], Ul[NT];
            f32x4 U[NT];
#pragma unroll
            for (int mm = 0; mm < NT; ++mm) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int n = 0; n < mm; ++n)
                    acc = h16::mma16(h16::tr4(&st.LT[strict_index(mm, n)][tro]), Uh[n], acc);
                f16x4 rh, rl;
                h16::split4(Y[mm] - acc, rh, rl);
                const f16x4 aa = h16::tr4(&st.InvT[mm][tro]);
                f32x4 uu = h16::mma16(aa, rh, f32x4{0.f, 0.f, 0.f, 0.f});
                uu = h16::mma16(aa, rl, uu);
                U[mm] = uu;
                h16::split4(uu, Uh[mm], Ul[mm]);
            }

            // O = (Gamma.Q) S + A_qk U, stored straight from the accumulators
            const bool full = (c + 1) * C <= T;
            const auto orr = rsrc(o_head + (size_t)c * C * Hdv);
            auto store_o = [&](int row, float x) {
                if constexpr (OBF)
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), orr, lane_v * 2u, (uint32_t)row * o_stride, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), orr, lane_v * 4u, (uint32_t)row * o_stride, 0);
            };
#pragma unroll
            for (int mm = 0; mm < NT; ++mm) {
                f32x4 acc = accQ[mm];
#pragma unroll
                for (int n = 0; n <= mm; ++n) {
                    const f16x4 aa = h16::tr4(&st.AqkT[lower_index(mm, n)][tro]);
                    acc = h16::mma16(aa, Uh[n], acc);
                    acc = h16::mma16(aa, Ul[n], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = c * C + TILE * mm + 4 * gq + i;
                    if (o && (full || t < T))
                        store_o(TILE * mm + i, acc[i]);
                }
            }

            // S <- Diag(Gamma_C) S + K-bar^T U; K-bar^T read transposed from its token rows
            // U's two fp16 terms as 8-item B operands (k-items: tokens of tiles 2j2 and 2j2 + 1)
            f16x8 Ubh[2], Ubl[2];
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2) {
                Ubh[j2] = __builtin_shufflevector(Uh[2 * j2], Uh[2 * j2 + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                Ubl[j2] = __builtin_shufflevector(Ul[2 * j2], Ul[2 * j2 + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            }
            const int tk = h16::tr_offset(lane, LDKB);
            static_assert(KT % 4 == 0, "row tiles of the state come in fours");
            f32x4 gam[4];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                if (kt % 4 == 0) row_gather16(st.GamC[16 * (kt + (r >> 2)) + 4 * gq + (r & 3)], gam);
                f32x4 acc = S[kt] * gam[kt % 4];
#pragma unroll
                for (int j2 = 0; j2 < 2; ++j2) {
                    const _Float16 *base = &st.Kb[(32 * j2) * LDKB + 16 * kt + tk];
                    const f16x4 a0 = h16::tr4(base);
                    const f16x4 a1 = h16::tr4(base + 16 * LDKB);
                    const f16x8 aa = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc = h16::mma32(aa, Ubh[j2], acc);
                    acc = h16::mma32(aa, Ubl[j2], acc);
                }
                S[kt] = acc;
            }
        }

        // the next chunk's slot is in LDS (every wave waited for its share)
        wait_vm();
        lds_barrier();
        failed = ss.failed != 0u;
        if (c + 1 < nchunks && w == 0 && lane == 0)
            post64(&consumed[((c + 1) % RING) * MAXSTATE + jst], tag(epoch, failed ? FAILED : (uint32_t)(c + 2)));
#pragma unroll
        for (int mm = 0; mm < NT; ++mm)
#pragma unroll
            for (int i = 0; i < 4; ++i) vin[mm][i] = vnx[mm][i];
    }
    if (failed && w == 0 && lane == 0) {
        // release the prep side from every slot wait
        for (int sl = 0; sl < RING; ++sl) post64(&consumed[sl * MAXSTATE + jst], tag(epoch, FAILED));
    }
    if (active && a.S_final) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.S_final[s_base + (size_t)(16 * kt + 4 * gq + i) * dv] = S[kt][i];
    }
}

// ------------------------------------------------------------------ host side

// Epochs start at a value drawn from the clock and the process, so a
// workspace that still holds flags written by another process is unlikely to
// hold this launch's epoch.
uint32_t epoch_seed() {
    uint64_t x = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    x ^= (uint64_t)getpid() << 32;
    x ^= (uint64_t)(uintptr_t)&x;
    x *= 0x9E3779B97F4A7C15ull;   // mix the bits (Fibonacci hashing)
    return (uint32_t)(x >> 32);
}
std::atomic<uint32_t> g_epoch{epoch_seed()};

uint32_t next_epoch() {
    uint32_t e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    while (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;   // 0 never tags a flag
    return e;
}

int nstate_for(int dv) { return (dv + SCOLS - 1) / SCOLS; }

template <int DK>
size_t slot_bytes() { return sizeof(Slot<DK>); }

// Heads per launch: every workgroup of a launch must be resident at once (one
// workgroup per CU at this LDS size), and a head's 1 + nstate workgroups are
// spread as 8 heads per (1 + nstate) x 8 block indices.
int group_heads(int resident, int nstate) {
    const int P = 1 + nstate;
    const int per8 = resident / (8 * P);
    return min(PS_MAX_GROUP, 8 * per8);
}

template <int DK, bool GBF, bool OBF, bool GL>
const void *kernel_ptr() { return reinterpret_cast<const void *>(&kda_chunk_ps_kernel<DK, GBF, OBF, GL>); }

// Workgroups the device can keep resident for this kernel (cached per device).
int resident_workgroups(const void *kern) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int ncu = 0, per = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, NTHREADS, 0) != hipSuccess) return 0;
    const int n = ncu * per;
    if (dev < 64 && n > 0) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

std::atomic<unsigned> g_spin_limit{1u << 20};

template <int DK, bool GBF, bool OBF, bool GL>
hipError_t launch(const ChunkFwdArgs &ca, void *ws, size_t ws_bytes, hipStream_t stream, bool &used)
{
    used = false;
    const void *kern = kernel_ptr<DK, GBF, OBF, GL>();
    const int nstate = nstate_for(ca.dv);
    const int BH = ca.B * ca.H;
    const int G = min(group_heads(resident_workgroups(kern), nstate), BH);
    if (G <= 0) return hipSuccess;   // not resident together: the caller takes the other kernel
    const size_t slot_off = ((size_t)G * FLAG_BYTES + 255) & ~(size_t)255;
    const size_t need = slot_off + (size_t)G * RING * sizeof(Slot<DK>);
    if (!ws || ws_bytes < need) return hipSuccess;
    used = true;
    PsArgs a;
    a.q = (const uint16_t *)ca.q; a.k = (const uint16_t *)ca.k; a.v = (const uint16_t *)ca.v;
    a.g = ca.g; a.beta = ca.beta; a.S0 = ca.S0; a.o = ca.o; a.S_final = ca.S_final; a.A_log = ca.A_log;
    a.ws = (unsigned char *)ws; a.slot_off = slot_off;
    a.B = ca.B; a.T = ca.T; a.H = ca.H; a.dv = ca.dv; a.nstate = nstate;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    (void)hipGetLastError();
    for (int h0 = 0; h0 < BH; h0 += G) {
        a.h_begin = h0;
        a.G = min(G, BH - h0);
        a.epoch = next_epoch();
        const unsigned grid = (unsigned)(8 * ((a.G + 7) / 8) * (1 + nstate));
        void *args[] = {&a};
        const hipError_t e = hipLaunchCooperativeKernel(kern, dim3(grid), dim3(NTHREADS), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, bool GL>
hipError_t dispatch(const ChunkFwdArgs &a, void *ws, size_t n, hipStream_t s, bool &used)
{
    if (a.gate_bf16)
        return a.out_bf16 ? launch<DK, true, true, GL>(a, ws, n, s, used) : launch<DK, true, false, GL>(a, ws, n, s, used);
    return a.out_bf16 ? launch<DK, false, true, GL>(a, ws, n, s, used) : launch<DK, false, false, GL>(a, ws, n, s, used);
}

}  // namespace

size_t chunk_ps_workspace_bytes(int B, int H, int dk, int dv)
{
    if (dk != 128 || dv <= 0 || dv % 64 != 0 || dv > 512 || B <= 0 || H <= 0) return 0;
    const int G = min(PS_MAX_GROUP, B * H);
    const size_t slot_off = ((size_t)G * FLAG_BYTES + 255) & ~(size_t)255;
    return slot_off + (size_t)G * RING * sizeof(Slot<128>);
}

hipError_t launch_chunk_fwd_ps(const ChunkFwdArgs &a, void *ws, size_t ws_bytes, hipStream_t stream, bool &used)
{
    used = false;
    if (!a.qkv_bf16 || a.dk != 128 || a.lengths || a.dv % 64 != 0 || a.dv > 512) return hipSuccess;
    // buffer offsets inside one chunk (64 rows of H * dv values) stay 32-bit
    if ((uint64_t)C * a.H * a.dv * 4 + (uint64_t)a.H * a.dv * 4 >= ((uint64_t)1 << 31)) return hipSuccess;
    return a.A_log ? dispatch<128, true>(a, ws, ws_bytes, stream, used) : dispatch<128, false>(a, ws, ws_bytes, stream, used);
}

unsigned set_spin_limit(unsigned limit)
{
    return g_spin_limit.exchange(limit, std::memory_order_relaxed);
}

unsigned spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

}  // namespace kda

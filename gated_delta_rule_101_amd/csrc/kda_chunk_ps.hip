// Chunkwise KDA forward for bfloat16 q, k, v on gfx950: the workgroups of a
// head share each chunk's state-independent work through a ring of chunk
// slots held in L2.
//
// The chunkwise form ("Kimi K3 - Lesson 3 of 14 - Sequence axis": sequential
// between chunks, parallel within; output = inter-chunk (Gamma . Q) S plus
// masked intra-chunk A V~; keys rescaled by 1/Gamma inside 16-token tiles,
// which the g_min = -5 floor keeps below e^80) splits into work that does not
// depend on the state (decays, scaled operands, Gram tiles, the diagonal
// inverses: everything a chunk needs before it meets S) and the state
// recurrence itself.  A head's dv columns are split into 64-column slabs, one
// workgroup each.  Every workgroup holds a prep team (four waves, one per
// 16-token tile) and four state waves (16 value columns each, the state slab
// in registers).  The prep teams of a head take turns: slab j prepares chunks
// j, j + nslab, ..., so each chunk's state-independent work is done once per
// head, not once per slab, and each CU carries an equal share of it.  A
// prepared chunk goes into one slot of a four-slot ring in the caller's
// workspace; the state waves of every slab copy the slot into LDS with
// LDS-direct loads one chunk ahead and then hand the slot back.  The ring is
// small (4 x 63 KB per head) and lives in the L2 of the XCD that runs the head.
//
// Synchronisation.  All workgroups of a head run on one XCD (workgroup i is
// dispatched to XCD i mod 8; each workgroup checks this at run time), so the
// XCD's L2 is the point where the workgroups meet: slot data and flags are
// written with ordinary stores (complete once s_waitcnt vmcnt(0) returns) and
// read with loads that bypass the CU's L1 (device scope, sc1).  Flags are
// 64-bit: the launch's epoch in the high half (a per-process counter, started
// at a random value and advanced per launch) and the chunk number + 1 in the
// low half; a wait accepts only the exact value it expects, so flags of other
// launches and uninitialised memory never satisfy it and the workspace needs
// no clearing.  Inside a workgroup the two roles never wait for each other:
// each role meets only its own four waves, at an LDS counter.  Every wait is
// bounded by `spin_limit` sleeps; when a bound expires the waiting side marks
// the launch failed (low half all ones), never overwrites a slot another
// workgroup may still read, and the state waves set their state to NaN, which
// carries into every output from then on and the final state: a failed launch
// is loud, and every wave still runs to its end.  The launch is cooperative,
// so all workgroups of the grid are resident together.
//
// Arithmetic and operand formats are those of kda_chunk_pipe.hip (the same
// producer and consumer steps, in the same order), so the two kernels give
// the same results.
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cstddef>
#include <mutex>

#include "kda_chunk_tiles.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

using namespace chunk;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NPROD = NT;             // prep waves: one per tile
constexpr int NSTW = 4;               // state waves: 16 value columns each
constexpr int NTHREADS = 64 * (NPROD + NSTW);
constexpr int SLAB = 16 * NSTW;       // value columns of one workgroup
constexpr int NSLOT = 4;              // ring slots per head
constexpr int MAXSLAB = 8;            // workgroups per head (dv <= 512)
constexpr size_t FLAG_BYTES = 1024;   // per head: ready line, consumed lines, info line
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

// Scratch of the prep team (LDS).
template <int DK>
struct alignas(16) TeamSmem {
    static constexpr int LDK = DK + 8;
    static constexpr int LDD = DK + 16;     // rows 64 bytes longer than DK floats (bank spread of the gathers)
    // Keys of tiles 0..2 decayed to their tile end.  Before that, entry m holds
    // tile m's gates staged for the transposed read of the in-tile cumulative
    // sum (entry 3 serves only that).
    _Float16 Kh[NT][TILE * LDK];
    float D[NT][LDD];                       // total decay of each tile
    float LdT[NT][TILE][TILE + 4];          // diagonal blocks of L (fp32): [m][col][row], 80-byte rows
    float betas[C];                         // beta of the chunk being prepared
    unsigned arrivals;                      // team meeting counter
    unsigned go;                            // leader's verdict on the slot wait (1: proceed)
};

template <int DK>
struct alignas(16) PsSmem {
    Slot<DK> stage[2];                      // the state waves' copies of two consecutive chunks
    TeamSmem<DK> team;
    unsigned state_arrivals;                // state waves' meeting counter
    unsigned failed;                        // set by any state wave whose wait expired
};
static_assert(sizeof(PsSmem<128>) <= 160 * 1024, "LDS budget of one workgroup");
static_assert(offsetof(Slot<128>, AqkT) % 16 == 0 && offsetof(Slot<128>, GamC) % 16 == 0 &&
              offsetof(Slot<128>, Kb) % 16 == 0 && offsetof(Slot<128>, beta) % 16 == 0, "slot alignment");
static_assert(offsetof(TeamSmem<128>, D) % 16 == 0 && offsetof(TeamSmem<128>, LdT) % 16 == 0 &&
              offsetof(TeamSmem<128>, betas) % 16 == 0, "team alignment");
static_assert((128 / 16) * TILE * LDT <= TILE * (128 + 8), "a tile's staged gates fit its key entry");

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
// The same load without making the value uniform: issue it early, take
// uniform() of the result where it is used, so nothing waits for it sooner.
__device__ __forceinline__ uint64_t poll64_raw(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void post64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every vector-memory access of this wave issued so far has completed (for
// stores: reached the L2).  The builtin form (vmcnt 0; expcnt and lgkmcnt at
// their "no wait" maxima) lets the compiler's wait-count tracking see it, so it
// adds no further waits for the same accesses later.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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
    int B, T, H, dv, nslab, h_begin, G;
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

    __shared__ PsSmem<DK> sm;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;     // row / column inside a 16x16 tile
    const int gq = lane >> 4;    // lane group: k-items, or output rows 4gq..4gq+3

    // Workgroup -> (head, slab).  Workgroup i runs on XCD i mod 8; the nslab
    // workgroups of a head are i = 8 (u nslab + slab) + x, all on XCD x.
    const int nslab = a.nslab;
    const int x = blockIdx.x & 7, s = blockIdx.x >> 3;
    const int u = s / nslab, slab = s - u * nslab;
    const int hl = u * 8 + x;   // head within this launch's group
    if (hl >= a.G) return;
    const int bh = a.h_begin + hl;
    const int b = bh / a.H, h = bh % a.H;
    const int T = a.T, H = a.H, dv = a.dv;
    const int nchunks = (T + C - 1) / C;
    const uint32_t epoch = a.epoch;
    const unsigned limit = a.spin_limit;

    uint64_t *flags = reinterpret_cast<uint64_t *>(a.ws + (size_t)hl * FLAG_BYTES);
    uint64_t *ready = flags;              // [NSLOT], written by the workgroup that prepared the slot
    uint64_t *consumed = flags + 16;      // [NSLOT][MAXSLAB], written by each workgroup's state waves
    uint64_t *info = flags + 64;          // [MAXSLAB]: each workgroup's XCD, tagged with the epoch
    SL *slots = reinterpret_cast<SL *>(a.ws + a.slot_off) + (size_t)hl * NSLOT;

    if (threadIdx.x == 0) {
        sm.team.arrivals = 0;
        sm.state_arrivals = 0;
        sm.failed = 0;
        post64(&info[slab], tag(epoch, xcc_id()));
    }
    __syncthreads();

    if (wave < NPROD) {
        // ====================================================== prep team
        const GT *g = static_cast<const GT *>(a.g);
        const GT *beta = static_cast<const GT *>(a.beta);
        const int m = wave;          // tile
        const bool leader = m == 0;
        TeamSmem<DK> &ts = sm.team;
        const float gate_scale = GL ? __expf(a.A_log[h]) : 1.f;

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
        // One loop instance per tile: the tile's work, and which of its values
        // stay live through the loop, are fixed at compile time.
        auto tile_loop = [&](auto tile) __attribute__((always_inline)) {
        constexpr int M = decltype(tile)::value;
        // this workgroup prepares chunks slab, slab + nslab, ...
        if (slab < nchunks) {
            load_g(slab);
            load_qk(slab);
            if (m == 0) bnext = load_beta(slab);
        }
        for (int cn = slab; cn < nchunks && ok; cn += nslab) {
            // Nothing is in flight here (the previous chunk ended with wait_vm);
            // saying so lets the compiler's wait tracking treat this chunk's
            // inputs as arrived, so it never waits for the prefetches issued below.
            wait_vm();
            const int slot = cn % NSLOT;
            SL *st = slots + slot;
            int r = lane & 15, gq = lane >> 4;
            asm volatile("" : "+v"(r), "+v"(gq));
            const bool live = cn * C + TILE * m + r < T;   // else: identity token
            const int cnext = cn + nslab < nchunks ? cn + nslab : cn;
            const uint64_t want = tag(epoch, (uint32_t)(cn - NSLOT + 1));

            // ---------------------------------------------- decays within tile m
            float f[KT][4];   // f = e^b in [e^-80, 1]
            if constexpr (GBF && !GL) {
                uint16_t *gs = reinterpret_cast<uint16_t *>(&ts.Kh[m][0]);
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

            if constexpr (M < NT - 1) {
#pragma unroll
                for (int blk = 0; blk < KT; ++blk) {
                    const int ch = 16 * blk + 4 * gq;
                    float kv[4];
                    in.k[blk].to_f32(kv);
                    f32x4 kh;
                    // the tile's total decay of these channels is lane 15's f in this row
#pragma unroll
                    for (int i = 0; i < 4; ++i) kh[i] = kv[i] * fast_rcp(f[blk][i]) * row_bcast<15>(f[blk][i]);
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
                if (cn >= NSLOT)
                    for (int j = 0; j < nslab; ++j)
                        wait_flag(&consumed[slot * MAXSLAB + j], want, tag(epoch, FAILED),
                                  poll64(&consumed[slot * MAXSLAB + j]), limit, free_ok);
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
                // the four tiles' totals of this lane's channels: one LDS read per
                // channel block, all issued before the first is used
                float dsrc[KT];
#pragma unroll
                for (int blk = 0; blk < KT; ++blk) dsrc[blk] = ts.D[r >> 2][16 * blk + 4 * gq + (r & 3)];
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int p = 0; p < KB; ++p) {
                    float qf[8], kf[8], ki[8], v2[8], v3[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int blk = 2 * p + hh;
                        const int ch = 16 * blk + 4 * gq;
                        f32x4 Dt[NT];
                        row_gather16(dsrc[blk], Dt);
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
            block_row(TileIndex<M>{});
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
        };
        static_assert(NT == 4, "one loop instance per tile");
        switch (m) {
        case 0: tile_loop(TileIndex<0>{}); break;
        case 1: tile_loop(TileIndex<1>{}); break;
        case 2: tile_loop(TileIndex<2>{}); break;
        default: tile_loop(TileIndex<3>{}); break;
        }
        if (!ok && leader && lane == 0) {
            // a wait expired: the state side stops waiting and writes NaN
            for (int sl = 0; sl < NSLOT; ++sl) post64(&ready[sl], tag(epoch, FAILED));
        }
        return;
    }

    // ========================================================== state waves
    const int w = wave - NPROD;
    const int col0 = SLAB * slab + 16 * w;        // first value column of this wave
    const int tid = (int)threadIdx.x - 64 * NPROD; // thread index among the state waves
    const size_t s_base = (size_t)bh * DK * dv + col0 + r;
    const size_t Hdv = (size_t)H * dv;
    const uint32_t lane_v = (uint32_t)(4 * gq * H * dv + r);   // rows 4gq + i, column r
    OT *o = static_cast<OT *>(a.o);
    constexpr int NCOPYS = (SLOT_U4 + 64 * NSTW - 1) / (64 * NSTW);

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
        const uint4 *src = reinterpret_cast<const uint4 *>(slots + c % NSLOT);
        const unsigned base = (unsigned)(size_t)&sm.stage[c & 1];
#pragma unroll
        for (int u2 = 0; u2 < NCOPYS; ++u2) {
            const int idx = u2 * 64 * NSTW + tid;
            const unsigned dst = __builtin_amdgcn_readfirstlane(base + (unsigned)(u2 * 64 * NSTW + 64 * w) * 16u);
            if (idx < SLOT_U4) lds_dma16(src + idx, dst);
        }
    };
    // this wave's verdict on chunk c's slot: ready, the prep side has not
    // failed, and (first chunk of each preparing workgroup) that workgroup
    // runs on this XCD
    auto slot_ok = [&](int c, uint64_t first) -> bool {
        bool ok = true;
        const uint64_t seen =
            wait_flag(&ready[c % NSLOT], tag(epoch, (uint32_t)(c + 1)), tag(epoch, FAILED), first, limit, ok);
        if (c < nslab && poll64(&info[c]) != tag(epoch, xcc_id())) ok = false;
        return ok && (uint32_t)seen != FAILED;
    };
    unsigned smeet = 0;   // state-wave meetings so far
    auto state_meet = [&]() {
        smeet += 1;
        if (!lds_meet(&sm.state_arrivals, NSTW * smeet, lane, limit) && lane == 0) sm.failed = 1u;
    };

#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[kt][i] = a.S0 ? a.S0[s_base + (size_t)(16 * kt + 4 * gq + i) * dv] : 0.f;

    bool failed = false;
    uint64_t pend = 0;   // polled value of the next chunk's ready flag (per lane, made uniform at use)
    if (nchunks > 0) {
        const bool okc = slot_ok(0, poll64(&ready[0]));
        if (okc) copy_slot(0);
        else if (lane == 0) sm.failed = 1u;
        load_v(0, vin);
        if (nchunks > 1) pend = poll64_raw(&ready[1 % NSLOT]);
    }
    wait_vm();
    state_meet();
    failed = __builtin_amdgcn_readfirstlane(sm.failed) != 0u;
    if (nchunks > 0 && w == 0 && lane == 0)
        post64(&consumed[0 * MAXSLAB + slab], tag(epoch, failed ? FAILED : 1u));

    // One chunk of the recurrence.  vcur holds this chunk's V; the next
    // chunk's V goes into vnext.  LDS operands are
    // read ahead of the products that use them: the state-independent tiles
    // first, each row tile's scaled queries and keys while the previous row
    // tile's products run, K-bar during the output products.  Scheduling fences
    // keep the compiler from sinking the reads back next to their uses.
    auto chunk_step = [&](int c, uint16_t (&vcur)[NT][4], uint16_t (&vnext)[NT][4]) __attribute__((always_inline)) {
        wait_vm();   // already true at run time (see the prep loop); for the compiler's wait tracking
        if (c + 1 < nchunks) {
            if (!failed) {
                const bool okc = slot_ok(c + 1, uniform64(pend));
                if (okc) copy_slot(c + 1);
                else if (lane == 0) sm.failed = 1u;
            }
            load_v(c + 1, vnext);
            if (!failed && c + 2 < nchunks) pend = poll64_raw(&ready[(c + 2) % NSLOT]);
        }
        const SL &st = sm.stage[c & 1];
        if (failed) {
            // this chunk's stage was not filled: the state turns NaN, and with it
            // every output from here on and the final state
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) S[kt] = f32x4{1.f, 1.f, 1.f, 1.f} * __builtin_nanf("");
        }
        const int tro = tile_tr_offset(lane);

        // ---- operands that do not depend on the state
        f16x4 lt[NSTRICT], inv[NT];
#pragma unroll
        for (int i = 0; i < NSTRICT; ++i) lt[i] = h16::tr4(&st.LT[i][tro]);
#pragma unroll
        for (int mm = 0; mm < NT; ++mm) inv[mm] = h16::tr4(&st.InvT[mm][tro]);
        f32x4 bts[NT];
        row_gather16(st.beta[TILE * (r >> 2) + 4 * gq + (r & 3)], bts);
        // scaled queries and keys of row tile mm: k-items channels 32j + 4gq + i and 32j + 16 + 4gq + i
        f16x8 aq[2][KB], ak[2][KB];
        auto load_rows = [&](int mm, f16x8 (&q8)[KB], f16x8 (&k8)[KB]) {
            const int row = (TILE * mm + r) * LDK;
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int ch = row + 32 * j + 4 * gq;
                q8[j] = h16::lds4x2(&st.Qt[ch], &st.Qt[ch + 16]);
                k8[j] = h16::lds4x2(&st.Kt[ch], &st.Kt[ch + 16]);
            }
        };
        load_rows(0, aq[0], ak[0]);

        // state slab as fp16 B operands
        f16x8 Sh[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) Sh[j] = h16::pack8(S[2 * j], S[2 * j + 1]);

        // ---- (Gamma.Q) S, computed transposed (the state slab as A operand,
        // the scaled queries as B): lane (g, r) then holds output columns
        // 4g..4g+3 of token r, four consecutive floats for one wide store;
        // and Y = beta (V - (Gamma.K) S) in the state's own layout
        f32x4 accQ[NT], Y[NT];
#pragma unroll
        for (int mm = 0; mm < NT; ++mm) {
            if (mm + 1 < NT) load_rows(mm + 1, aq[(mm + 1) & 1], ak[(mm + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 aQ = {0.f, 0.f, 0.f, 0.f}, aK = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                aQ = h16::mma32(Sh[j], aq[mm & 1][j], aQ);
                aK = h16::mma32(ak[mm & 1][j], Sh[j], aK);
            }
            accQ[mm] = aQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) Y[mm][i] = bts[mm][i] * (to_f32(vcur[mm][i]) - aK[i]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- A_qk tiles, read while the solve runs
        f16x4 aqk[NLOWER];
#pragma unroll
        for (int i = 0; i < NLOWER; ++i) aqk[i] = h16::tr4(&st.AqkT[i][tro]);

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

        // ---- K-bar^T operands of the first four state row tiles, read during the output products
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
        f32x4 gam[KT / 4][4];
        static_assert(KT % 4 == 0, "row tiles of the state come in fours");
#pragma unroll
        for (int q4 = 0; q4 < KT / 4; ++q4) row_gather16(st.GamC[16 * (4 * q4 + (r >> 2)) + 4 * gq + (r & 3)], gam[q4]);
        __builtin_amdgcn_sched_barrier(0);

        // ---- O^T = ((Gamma.Q) S)^T + U^T A_qk^T (U as the A operand, the A_qk
        // tiles as B): lane (g, r) holds four consecutive columns of token r,
        // one wide store per row tile
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
            if (o && c * C + TILE * mm + r < T) {
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

        // the next chunk's slot is in LDS (every state wave waited for its share)
        wait_vm();
        state_meet();
        failed = __builtin_amdgcn_readfirstlane(sm.failed) != 0u;
        if (c + 1 < nchunks && w == 0 && lane == 0)
            post64(&consumed[((c + 1) % NSLOT) * MAXSLAB + slab], tag(epoch, failed ? FAILED : (uint32_t)(c + 2)));
    };
    for (int c = 0; c < nchunks; ++c) {
        chunk_step(c, vin, vnx);
#pragma unroll
        for (int mm = 0; mm < NT; ++mm)
#pragma unroll
            for (int i = 0; i < 4; ++i) vin[mm][i] = vnx[mm][i];
    }
    if (failed && w == 0 && lane == 0) {
        // release every prep team from its slot waits
        for (int sl = 0; sl < NSLOT; ++sl) post64(&consumed[sl * MAXSLAB + slab], tag(epoch, FAILED));
    }
    if (a.S_final) {
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

int nslab_for(int dv) { return dv / SLAB; }

template <int DK>
size_t slot_bytes() { return sizeof(Slot<DK>); }

// Heads per launch: every workgroup of a launch must be resident at once (one
// workgroup per CU at this LDS size), and a head's nslab workgroups are
// spread as 8 heads per nslab x 8 block indices.
int group_heads(int resident, int nslab) {
    const int per8 = resident / (8 * nslab);
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
    const int nslab = nslab_for(ca.dv);
    const int BH = ca.B * ca.H;
    const int G = min(group_heads(resident_workgroups(kern), nslab), BH);
    if (G <= 0) return hipSuccess;   // not resident together: the caller takes the other kernel
    const size_t slot_off = ((size_t)G * FLAG_BYTES + 255) & ~(size_t)255;
    const size_t need = slot_off + (size_t)G * NSLOT * sizeof(Slot<DK>);
    if (!ws || ws_bytes < need) return hipSuccess;
    used = true;
    PsArgs a;
    a.q = (const uint16_t *)ca.q; a.k = (const uint16_t *)ca.k; a.v = (const uint16_t *)ca.v;
    a.g = ca.g; a.beta = ca.beta; a.S0 = ca.S0; a.o = ca.o; a.S_final = ca.S_final; a.A_log = ca.A_log;
    a.ws = (unsigned char *)ws; a.slot_off = slot_off;
    a.B = ca.B; a.T = ca.T; a.H = ca.H; a.dv = ca.dv; a.nslab = nslab;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    (void)hipGetLastError();
    for (int h0 = 0; h0 < BH; h0 += G) {
        a.h_begin = h0;
        a.G = min(G, BH - h0);
        a.epoch = next_epoch();
        const unsigned grid = (unsigned)(8 * ((a.G + 7) / 8) * nslab);
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

// The ring of the no-allocation entry point: file-scope device memory, one
// copy per device, held until the process ends.  Host code reaches it only
// through the per-device address that hipGetSymbolAddress returns (the
// array's name on the host is a stand-in, not a device address).
constexpr size_t NOALLOC_BYTES =
    (((size_t)NOALLOC_HEADS * FLAG_BYTES + 255) & ~(size_t)255) + (size_t)NOALLOC_HEADS * NSLOT * sizeof(Slot<128>);
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return NOALLOC_BYTES; }

hipError_t noalloc_scratch(hipStream_t stream, void **out)
{
    *out = nullptr;
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (stream && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // looked up once per device, with that device current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t chunk_ps_workspace_bytes(int B, int H, int dk, int dv)
{
    if (dk != 128 || dv < 2 * SLAB || dv % SLAB != 0 || dv > SLAB * MAXSLAB || B <= 0 || H <= 0) return 0;
    const int G = min(PS_MAX_GROUP, B * H);
    const size_t slot_off = ((size_t)G * FLAG_BYTES + 255) & ~(size_t)255;
    return slot_off + (size_t)G * NSLOT * sizeof(Slot<128>);
}

hipError_t launch_chunk_fwd_ps(const ChunkFwdArgs &a, void *ws, size_t ws_bytes, hipStream_t stream, bool &used)
{
    used = false;
    // one slab per head shares nothing: the ring would only add its copies
    if (!a.qkv_bf16 || a.dk != 128 || a.lengths || a.dv < 2 * SLAB || a.dv % SLAB != 0 || a.dv > SLAB * MAXSLAB)
        return hipSuccess;
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

// Fused forward: the intra-chunk stage and the inter-chunk scan in one
// persistent kernel whose hand-off records never leave the XCD that makes
// and consumes them.
//
// Why.  The FlashKDA write-up splits the forward into a token-parallel
// kernel and a low-parallelism scan and reports that the split beat its
// fused prototype ("Moonshot AI Open-Sources FlashKDA", section "What makes
// the kernel fast").  On MI355X the split costs more than it does there: the
// records (864 B per token and head at 32-token chunks, more than half the
// algorithmic 1282 B) then cross the fabric between the XCDs and memory
// twice, and the fabric carries about 7 TB/s whether the bytes come from HBM
// or from the memory-side cache.  Here both stages share the chip instead:
//
//   * Units.  A unit is one (sequence, head); unit u lives on XCD u mod 8
//     (workgroups are dispatched to the XCDs round robin, so workgroup b
//     runs on XCD b mod 8).  Every unit has a ring of RG record slots in
//     global memory, which stays in that XCD's L2.
//   * Scan parts.  A unit's 128 state columns are split into parts of 64;
//     workgroup i of an XCD scans part i mod PP of unit i / PP of that XCD
//     with four waves of 16 columns, the state in MFMA accumulators, as the
//     two-kernel scan does.
//   * Intra waves.  The intra waves of all of an XCD's workgroups make the
//     records of the XCD's units, chunk by chunk across the units (item
//     k -> chunk k / U, unit k mod U), each into its unit's ring slot.
//   * A loader wave copies each record from the L2 ring into an LDS ring
//     (buffer-to-LDS DMA that bypasses the vector L1) for the scan waves; a
//     poller wave mirrors the ring's ready flags into LDS and publishes how
//     far the workgroup has copied, which frees ring slots for producers.
//
// Flags are 32-bit counters in global memory, read and written with
// agent-scope atomics (coherent across the whole device), zeroed by a small
// kernel before each launch.  A record's plain stores complete (s_waitcnt)
// before its ready flag is set, and its readers run on the same XCD, hence
// read the same L2.  No wave waits on a later item than one it already
// waits for, so the waits always end: the earliest waiting item needs only
// records of earlier items, which are either done or being made.  Every
// wait is also bounded (about a second); a wait that runs out sets an error
// word and lets the kernel finish.  The launch is cooperative, so all
// workgroups are resident at once.
#include <stdlib.h>

#include "kda_c32_dev.h"
#include "kda_launch.h"
#include "kda_team_dev.h"

namespace kda {

namespace {

constexpr int FW_SCAN = 4;                 // scan waves (16 columns each)
constexpr int FW_LOADER = 4;               // record DMA wave
constexpr int FW_POLLER = 5;               // global <-> LDS flag wave
constexpr int FW_INTRA0 = 6;               // first wave of the intra teams
constexpr int FW_TEAMS = 2;                // teams of four waves
constexpr int FW_WAVES = FW_INTRA0 + 4 * FW_TEAMS;
constexpr int PART_CW = 64;                // columns per scan part
constexpr int RG = 8;                      // record slots per unit in the L2 ring
constexpr int RL = 3;                      // LDS ring slots
constexpr int SLOT_BYTES = Rec32::BYTES;
constexpr int REC_UNITS = Rec32::BYTES / 1024;   // 1 KB DMAs per record
constexpr int NFLAGS = RG + 2;             // per unit: ready[RG], consumed[2]
// Bounds of the waits: global flag polls take a memory round trip (about a
// microsecond), LDS polls tens of cycles; both bounds are around a second.
constexpr uint32_t MAX_GPOLLS = 1u << 20;
constexpr uint32_t MAX_LPOLLS = 1u << 23;

struct FusedArgs {
    const uint16_t *q, *k, *v, *g, *beta;
    const float *A_log, *dt_bias;
    float lb2, scale;
    const int32_t *cu;
    int N, T, H, K;                        // K = V: 128, or 64 on the 128-wide tiles
    const void *init;
    int init_fp32;
    void *fin;
    int fin_fp32;
    uint16_t *out;
    uint8_t *ring;                         // units x RG x SLOT_BYTES
    uint32_t *flags;                       // units x NFLAGS, zero at launch; then the error word
    int nchmax;                            // chunks of the longest possible sequence
};

struct alignas(16) FusedLds {
    uint8_t ring[RL][Rec32::BYTES];
    int lready[RL];                        // landings per slot (one per use)
    int lfree[RL];                         // scan-wave releases per slot (four per use)
    int gready;                            // chunks whose records are ready in the L2 ring
    int lcons;                             // chunks copied into the LDS ring
    TeamLds team[FW_TEAMS];
};

__device__ __forceinline__ uint32_t flag_load(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// LDS flags between the waves of a workgroup: acquire loads, release
// stores and adds (ordering for the compiler; LDS itself is coherent).
__device__ __forceinline__ int lds_load(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(int *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Adds v once for the wave (from its first lane: an add made by all 64
// lanes would count 64 times).
__device__ __forceinline__ void lds_add(int *p, int v) {
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until *p >= want (LDS); false if the wait ran out.
__device__ __forceinline__ bool wait_lds_ge(const int *p, int want) {
    for (uint32_t n = 0; n < MAX_LPOLLS; ++n) {
        if (lds_load(p) >= want) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t rsrc_words_f(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    i32x4_t r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}
// 16-byte-per-lane buffer-to-LDS DMA that misses in the vector L1 (sc0): the
// ring slot was written by another compute unit of the XCD, so only L2 has
// it.  Waits are explicit (the loader's vmcnt ladder).
__device__ __forceinline__ void dma16_sc0(i32x4_t rs, const void *lds, int off) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen sc0 lds"
                 :: "s"(m0), "v"(off), "s"(rs) : "memory", "m0");
}

template <int SRC>
__device__ __forceinline__ float row_bcast_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              0x150 + SRC, 0xf, 0xf, true));
}
template <int T, int J>
__device__ __forceinline__ float decay_f(const float (&gm)[2]) {
    return row_bcast_f<4 * (T >> 1) + 2 * (T & 1) + (J >> 1)>(gm[J & 1]);
}
template <int T>
__device__ __forceinline__ void decay_tiles_f(f32x4_t (&S)[8], const float (&gm)[2]) {
    if constexpr (T < 8) {
        S[T][0] *= decay_f<T, 0>(gm);
        S[T][1] *= decay_f<T, 1>(gm);
        S[T][2] *= decay_f<T, 2>(gm);
        S[T][3] *= decay_f<T, 3>(gm);
        decay_tiles_f<T + 1>(S, gm);
    }
}

__global__ void zero_flags_kernel(uint32_t *__restrict__ p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// VD: head dimension (128, or 64 on the 128-wide tiles); PP = VD / 64 scan
// parts per unit.  SG: the Gated DeltaNet form (g [B*T, H], dt_bias [H]).
template <int VD, bool SG>
__global__ __launch_bounds__(64 * FW_WAVES, 1) void fused_kernel(FusedArgs a)
{
    constexpr int K = VD, V = VD;
    constexpr int PP = V / PART_CW;
    __shared__ FusedLds L;

    const int b = blockIdx.x;
    const int x = b & 7;                               // XCD (round-robin dispatch)
    const int wi = b >> 3;                             // workgroup index on the XCD
    const int Q = (int)(gridDim.x >> 3);
    const int NH = a.N * a.H;
    const int Ux = NH > x ? (NH - x + 7) / 8 : 0;      // units u = x + 8m on this XCD
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int grp = l >> 4, cg = l & 15;
    uint32_t *err = a.flags + (size_t)NH * NFLAGS;

    if (threadIdx.x < RL) { L.lready[threadIdx.x] = 0; L.lfree[threadIdx.x] = 0; }
    if (threadIdx.x < 64 * FW_TEAMS && (threadIdx.x & 63) == 0) team_init(L.team[threadIdx.x >> 6]);
    if (threadIdx.x == 0) {
        L.gready = 0;
        L.lcons = 0;
        // records pass through the L2 of the XCD the workgroup runs on: the
        // round-robin placement this relies on is checked here
        const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 7u;  // HW_REG_XCC_ID[3:0]
        if ((int)xcc != x) flag_store(err, 5u);
    }
    __syncthreads();                                   // the only workgroup barrier

    // ---- intra teams: records of the XCD's units, chunk-major --------------
    if (w >= FW_INTRA0) {
        const int tw = w - FW_INTRA0;
        const int tm = tw >> 2, kb = tw & 3;           // team, its channel block
        TeamLds &T = L.team[tm];
        const int NT = Q * FW_TEAMS;                   // teams on the XCD
        const int64_t items = (int64_t)Ux * a.nchmax;
        bool ok = true;                                // false once a wait ran out: no more waits
        int done = 0;                                  // chunks this team has made
        for (int64_t kk = (int64_t)wi * FW_TEAMS + tm; kk < items; kk += NT) {
            const int j = (int)(kk / Ux);
            const int m = (int)(kk - (int64_t)j * Ux);
            const int u = x + 8 * m;
            const int n = u / a.H, h = u - n * a.H;
            int64_t start, end;
            seq_range(a.cu, n, a.T, start, end);
            const int64_t t0 = start + (int64_t)j * C32;
            if (t0 >= end) continue;                   // past this sequence's end (uniform in the team)
            const int len = (int)min((int64_t)C32, end - t0);
            uint32_t *fl = a.flags + (size_t)u * NFLAGS;
            const int gs = j % RG;
            if (ok && j >= RG) {                       // the slot's previous record copied by every part
                bool free_ = false;
                for (uint32_t p = 0; p < MAX_GPOLLS && !free_; ++p) {
                    const uint32_t c = (l < PP) ? flag_load(fl + RG + l) : 0xffffffffu;
                    uint32_t cmin = c;
#pragma unroll
                    for (int pp = 0; pp < PP; ++pp) cmin = min(cmin, (uint32_t)__builtin_amdgcn_readlane((int)c, pp));
                    free_ = cmin >= (uint32_t)(j - RG + 1);
                    if (!free_) __builtin_amdgcn_s_sleep(2);
                }
                if (!free_) { ok = false; flag_store(err, 1u); }
            }
            uint8_t *rec = a.ring + ((size_t)u * RG + gs) * SLOT_BYTES;
            const float A = expf(a.A_log[h]);
            ok = team_chunk<SG, false>(T, kb, done, a.q, a.k, a.g, a.beta, a.dt_bias, A, a.lb2, t0, len,
                                       a.H, h, a.K, rec) && ok;
            ++done;
            if (kb == 0) {
                // every wave's stores of the record acknowledged by L2
                ok = ok && team_wait(&T.p3, 4 * done);
                flag_store(fl + gs, (uint32_t)(j + 1));
            }
        }
        if (!ok) flag_store(err, 1u);
        return;
    }

    // ---- this workgroup's scan part -----------------------------------------
    const int m = wi / PP, part = wi - (wi / PP) * PP;
    if (m >= Ux) return;                               // no part here (uniform)
    const int u = x + 8 * m;
    const int n = u / a.H, h = u - n * a.H;
    int64_t start, end;
    seq_range(a.cu, n, a.T, start, end);
    const int64_t Lseq = end - start;
    const int nch = __builtin_amdgcn_readfirstlane((int)((Lseq + C32 - 1) / C32));
    uint32_t *fl = a.flags + (size_t)u * NFLAGS;
    const uint8_t *ring_u = a.ring + (size_t)u * RG * SLOT_BYTES;

    if (w == FW_POLLER) {
        // ready flags of the unit's ring (all RG in one load) -> L.gready;
        // L.lcons -> this part's consumed flag
        int ready = 0, published = 0;
        for (uint32_t p = 0; p < MAX_GPOLLS; ++p) {
            const uint32_t f = (l < RG) ? flag_load(fl + l) : 0u;
#pragma unroll
            for (int step = 0; step < RG; ++step) {
                const uint32_t fs = (uint32_t)__builtin_amdgcn_readlane((int)f, ready % RG);
                if (ready < nch && fs >= (uint32_t)(ready + 1)) ++ready;
            }
            lds_store(&L.gready, ready);
            const int c = lds_load(&L.lcons);
            if (c > published) { flag_store(fl + RG + part, (uint32_t)c); published = c; }
            if (ready == nch && published == nch) return;
            __builtin_amdgcn_s_sleep(1);
        }
        flag_store(err, 2u);
        return;
    }

    if (w == FW_LOADER) {
        // two chunks of record DMAs in flight (2 x 27 <= 63 in vmcnt)
        static_assert(2 * REC_UNITS <= 63, "vmcnt holds at most 63");
        bool ok = true;
        for (int j = 0; j < nch; ++j) {
            const int s = j % RL;
            if (ok && j >= RL) ok = wait_lds_ge(&L.lfree[s], FW_SCAN * (j / RL));
            if (ok) ok = wait_lds_ge(&L.gready, j + 1);
            const i32x4_t rr = rsrc_words_f(ring_u + (size_t)(j % RG) * SLOT_BYTES, ok ? (uint32_t)Rec32::BYTES : 0u);
            // The slot held an older record, which this compute unit may
            // still have in its vector L1 (coherent within the compute
            // unit, not across them): invalidate the L1 first (the
            // workgroup-scope acquire), then read the new record from L2.
            asm volatile("buffer_inv sc0" ::: "memory");
#pragma unroll
            for (int unit = 0; unit < REC_UNITS; ++unit) dma16_sc0(rr, &L.ring[s][unit * 1024], unit * 1024 + l * 16);
            if (j >= 1) {
                // chunk j-1 landed (whether or not the invalidate counts in vmcnt)
                asm volatile("s_waitcnt vmcnt(%0)" :: "n"(REC_UNITS) : "memory");
                lds_add(&L.lready[(j - 1) % RL], 1);
                lds_store(&L.lcons, j);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (nch > 0) {
            lds_add(&L.lready[(nch - 1) % RL], 1);
            lds_store(&L.lcons, nch);
        }
        if (!ok) flag_store(err, 3u);
        return;
    }

    // ---- scan waves -----------------------------------------------------------
    const int wcol0 = w * 16;
    const int col0 = part * PART_CW;
    const size_t row_bytes = (size_t)a.H * V * 2;
    f32x4_t S[8];
    {
        const size_t slab = (size_t)K * V * (a.init_fp32 ? 4 : 2);
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc((const uint8_t *)a.init + (a.init ? ((size_t)n * a.H + h) * slab : 0),
                      a.init ? (uint32_t)slab : 0u);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int idx = state_chan(t, 4 * grp + jj) * V + col0 + wcol0 + cg;
                S[t][jj] = a.init_fp32
                    ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4, 0, 0))
                    : bf16f(__builtin_amdgcn_raw_buffer_load_b16(rs, idx * 2, 0, 0));
            }
    }
    const size_t row_stride = (size_t)C32 * a.H * V;
    const uint16_t *v_base = a.v + ((size_t)start * a.H + h) * V + col0 + wcol0;
    uint16_t *out_base = a.out + ((size_t)start * a.H + h) * V + col0;
    // v of chunk c as the two A operands of the identity transposes: lane l
    // reads token 16rt + l%16, columns 4(l/16) .. +3 of this wave's slice
    auto load_v = [&](int c, u32x2_t (&vv)[2]) {
        const int64_t rem = Lseq - (int64_t)c * C32;
        const int len = (int)(rem < C32 ? rem : C32);
        const __amdgpu_buffer_rsrc_t rv =
            make_rsrc(v_base + (size_t)c * row_stride, (uint32_t)((len - 1) * row_bytes + 32));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
            vv[rt] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                rv, (int)((16 * rt + cg) * row_bytes) + 8 * grp, 0, 2));
    };
    const int gch = 32 * (cg >> 2) + 8 * grp + 4 * ((cg >> 1) & 1) + 2 * (cg & 1);
    auto lds16 = [&](const uint8_t *p) { return *(const u32x4_t *)p; };
    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;
        const int d = cg - 4 * grp;
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    const float scale = a.scale;
    u32x2_t vnext[2];
    if (nch > 0) load_v(0, vnext);
    bool ok = true;
    for (int c = 0; c < nch; ++c) {
        u32x2_t vcur[2] = {vnext[0], vnext[1]};
        if (c + 1 < nch) load_v(c + 1, vnext);
        const int s = c % RL;
        if (ok) ok = wait_lds_ge(&L.lready[s], c / RL + 1);
        const uint8_t *Rp = L.ring[s];
        const int64_t rem = Lseq - (int64_t)c * C32;
        const int len = (int)(rem < C32 ? rem : C32);
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(out_base + (size_t)c * row_stride, (uint32_t)((len - 1) * row_bytes + PART_CW * 2));
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        u32x4_t Sb[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            Sb[kb][0] = pack2(S[2 * kb][0], S[2 * kb][1]);
            Sb[kb][1] = pack2(S[2 * kb][2], S[2 * kb][3]);
            Sb[kb][2] = pack2(S[2 * kb + 1][0], S[2 * kb + 1][1]);
            Sb[kb][3] = pack2(S[2 * kb + 1][2], S[2 * kb + 1][3]);
        }
        // operands read from the LDS slot group by group, just before their
        // MFMAs (the whole set would not fit beside the intra waves' registers)
        f32x4_t P[2] = {zero, zero}, Qs[2] = {zero, zero}, vv[2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                P[rt] = mfma_k32(lds16(Rp + Rec32::KT + ((kb * 2 + rt) * 64 + l) * 16), Sb[kb], P[rt]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) vv[rt] = mfma_k16(vcur[rt], eye, zero);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                Qs[rt] = mfma_k32(lds16(Rp + Rec32::QT + ((kb * 2 + rt) * 64 + l) * 16), Sb[kb], Qs[rt]);
        float gm[2];
        {
            const u32x2_t g2 = *(const u32x2_t *)(Rp + Rec32::GAM + gch * 4);
            gm[0] = __uint_as_float(g2[0]);
            gm[1] = __uint_as_float(g2[1]);
        }
        decay_tiles_f<0>(S, gm);
        u32x4_t Xb;
        Xb[0] = pack2(vv[0][0] - P[0][0], vv[0][1] - P[0][1]);
        Xb[1] = pack2(vv[0][2] - P[0][2], vv[0][3] - P[0][3]);
        Xb[2] = pack2(vv[1][0] - P[1][0], vv[1][1] - P[1][1]);
        Xb[3] = pack2(vv[1][2] - P[1][2], vv[1][3] - P[1][3]);
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mfma_k32(lds16(Rp + Rec32::WT + (t * 64 + l) * 16), Xb, S[t]);
        f32x4_t MX[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) MX[rt] = mfma_k32(lds16(Rp + Rec32::M + (rt * 64 + l) * 16), Xb, zero);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's reads of the slot done
        lds_add(&L.lfree[s], 1);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const u32x2_t oa = {pack2(scale * (Qs[rt][0] + MX[rt][0]), scale * (Qs[rt][1] + MX[rt][1])),
                                pack2(scale * (Qs[rt][2] + MX[rt][2]), scale * (Qs[rt][3] + MX[rt][3]))};
            const f32x4_t ot = mfma_k16(oa, eye, zero);
            const u32x2_t os = {pack2(ot[0], ot[1]), pack2(ot[2], ot[3])};
            __builtin_amdgcn_raw_buffer_store_b64(
                os, ro, (int)((16 * rt + cg) * row_bytes) + (wcol0 + 4 * grp) * 2, 0, 0);
        }
    }
    if (!ok) flag_store(err, 4u);
    if (a.fin) {
        const size_t slab = (size_t)K * V * (a.fin_fp32 ? 4 : 2);
        const __amdgpu_buffer_rsrc_t rf =
            make_rsrc((uint8_t *)a.fin + ((size_t)n * a.H + h) * slab, (uint32_t)slab);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int idx = state_chan(t, 4 * grp + jj) * V + col0 + wcol0 + cg;
                if (a.fin_fp32)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[t][jj]), rf, idx * 4, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(tobf16(S[t][jj]), rf, idx * 2, 0, 0);
            }
    }
}

int fused_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

}  // namespace

size_t fused_workspace_bytes(int N, int H) {
    const size_t units = (size_t)N * H;
    return units * RG * SLOT_BYTES + (units * NFLAGS + 64) * sizeof(uint32_t);
}

// Whether all 8 Q workgroups of the kernel fit the device at once (one per
// compute unit), per device.
bool fused_resident() {
    static int cached[64];                 // 0 unknown, 1 yes, 2 no
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    if (!cached[dev]) {
        const int cus = fused_cus();
        int per_cu = 0;
        bool ok = cus >= 8 && cus % 8 == 0;
        const void *fns[4] = {(const void *)fused_kernel<HD, false>, (const void *)fused_kernel<64, false>,
                              (const void *)fused_kernel<HD, true>, (const void *)fused_kernel<64, true>};
        for (int f = 0; f < 4 && ok; ++f) {
            per_cu = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fns[f], 64 * FW_WAVES, 0) != hipSuccess ||
                per_cu < 1)
                ok = false;
        }
        (void)hipGetLastError();
        cached[dev] = ok ? 1 : 2;
    }
    return cached[dev] == 1;
}

// The fused path is taken when KDA_FUSED is set to a value other than "0"
// in the environment (read at each call).
bool fused_enabled() {
    const char *e = getenv("KDA_FUSED");
    return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

bool fused_applicable(int64_t tokens, int N, int H, int K) {
    if (!fused_enabled()) return false;
    if (K != HD && K != 64) return false;
    const int cus = fused_cus();
    if (cus < 8 || cus % 8 || !fused_resident()) return false;
    const int Q = cus / 8;
    const int64_t NH = (int64_t)N * H;
    const int PP = K / PART_CW;
    // every scan part resident at once: at most Q parts per XCD
    if ((NH + 7) / 8 * PP > Q) return false;
    return tokens > 0;
}

hipError_t launch_fused(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                        const uint16_t *beta, float scale, const float *A_log, const float *dt_bias,
                        float lower_bound, const int32_t *cu, int N, int T, int H, int K,
                        int64_t tokens, const void *init, int init_fp32, void *fin, int fin_fp32,
                        uint16_t *out, void *ws, hipStream_t stream, bool scalar_gate)
{
    const size_t units = (size_t)N * H;
    FusedArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.A_log = A_log; a.dt_bias = dt_bias;
    a.lb2 = lower_bound * LOG2E;
    a.scale = scale;
    a.cu = cu; a.N = N; a.T = T; a.H = H; a.K = K;
    a.init = init; a.init_fp32 = init_fp32; a.fin = fin; a.fin_fp32 = fin_fp32; a.out = out;
    a.ring = (uint8_t *)ws;
    a.flags = (uint32_t *)((uint8_t *)ws + units * RG * SLOT_BYTES);
    // the longest sequence has at most all tokens (fixed length: T)
    a.nchmax = (int)(((cu ? tokens : (int64_t)T) + C32 - 1) / C32);
    const int nflags = (int)(units * NFLAGS + 64);
    hipLaunchKernelGGL(zero_flags_kernel, dim3((nflags + 255) / 256), dim3(256), 0, stream,
                       a.flags, nflags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int Q = fused_cus() / 8;
    void *args[] = {&a};
    const void *fn = K == HD ? (scalar_gate ? (const void *)fused_kernel<HD, true> : (const void *)fused_kernel<HD, false>)
                             : (scalar_gate ? (const void *)fused_kernel<64, true> : (const void *)fused_kernel<64, false>);
    return hipLaunchCooperativeKernel(fn, dim3(8 * Q), dim3(64 * FW_WAVES), args, 0, stream);
}

const uint32_t *fused_error_word(const void *ws, int N, int H) {
    const size_t units = (size_t)N * H;
    return (const uint32_t *)((const uint8_t *)ws + units * RG * SLOT_BYTES) + units * NFLAGS;
}

}  // namespace kda

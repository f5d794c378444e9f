// The Newton-Schulz products' tiled NT GEMM on MFMA with eight wavefronts per
// workgroup (two per SIMD): the same LDS ring, operand swizzle and epilogue
// passes as the four-wavefront core in gemm_core.h, with each wavefront owning
// half as many accumulators.
//
// Why two waves per SIMD.  With one wavefront per SIMD, every stall of that
// wavefront's in-order instruction stream (a direct-to-LDS load waiting for a
// free slot in the CU's load queue, the stage barrier, the epilogue's LDS
// round trips, loads and stores) leaves the SIMD's matrix core idle; with two,
// the other wavefront's MFMAs fill some of those gaps.  Each wavefront holds a
// 128 x 64 (or 64 x 64) block of the tile in 128 accumulators, so a substep
// reads 6 fragments for 8 MFMAs instead of 8 for 16 (LDS reads go up by half,
// within the LDS bandwidth), and an epilogue operand is read from memory
// instead of being captured from the K loop (no registers left for it).
// Measured against the four-wavefront core on the workload buckets: 1-4 %
// faster per step, most of it in the epilogue-heavy last Update.
#pragma once

#include "gemm_core.h"

namespace mo_gemm {

constexpr int G8_THREADS = 512;

// Wave layout of a 256 x TN tile (TN = 64 NB; NB = 4 or 2) on 8 wavefronts:
// WM x WN wavefronts, each MB x NBW blocks of 32 x 32.
template <int NB> struct Layout8;
template <> struct Layout8<4> { static constexpr int WM = 2, WN = 4, MB = 4, NBW = 2; };
template <> struct Layout8<2> { static constexpr int WM = 4, WN = 2, MB = 2, NBW = 2; };

// One 256 x TN tile of C = P Q^T (TN = 64 NB), as gemm_core but on 8
// wavefronts.  Pm, Qm, ld, ti, tj and the epilogue object are as there; the
// epilogue must not ask for the captured operand (CAP) or a rotated K order.
template <typename T, int NB, class MakeEp>
__device__ __forceinline__ void gemm_core8(uint8_t* smem, const T* Pm, const T* Qm, int64_t ld, int ti,
                                           int tj, const MakeEp& make_ep) {
    using Ep = decltype(make_ep());
    static_assert(!Ep::CAP && !Ep::KROT, "the 8-wave core reads its epilogue operand from memory");
    using L = Layout8<NB>;
    constexpr int WM = L::WM, WN = L::WN, MB = L::MB, NBW = L::NBW;
    constexpr int TN = 64 * NB;                  // tile columns = rows of Q
    constexpr int SBYTES = OPND_BYTES + TN * KB; // one stage: P (256 rows) then Q (TN rows)
    constexpr int QROWS = TN / 8;                // Q rows each wave loads per stage
    constexpr int LS = 2 + QROWS / 16;           // load instructions per stage and wave
    constexpr int LP = 2 * LS;                   // ... per pair of stages
    constexpr int MF = MB * NBW;                 // MFMA blocks per wave and substep
    constexpr int NR = MB + NBW;                 // fragment reads per substep
    static_assert(QROWS % 16 == 0 && WM * WN == 8 && WM * MB * 32 == GT && WN * NBW * 32 == TN, "layout");
    static_assert(NSTAGE * SBYTES <= GEMM_LDS, "LDS ring");
    const T* P = Pm + int64_t(ti) * GT * ld;
    const T* Q = Qm + int64_t(tj) * TN * ld;
    const int64_t ldb = ld * int64_t(sizeof(T));
    const int nk = int(ldb / KB);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int r32 = lane & 31, kg = lane >> 5;

    // direct-to-LDS loads: wave w fills P rows [32 w, 32 w + 32) and Q rows
    // [QROWS w, QROWS (w + 1)), 16 rows (1 KB) per instruction; lane l -> row
    // + l / 4, physical chunk l % 4 (see gemm_core).
    const uint8_t* Pb = reinterpret_cast<const uint8_t*>(P);
    const uint8_t* Qb = reinterpret_cast<const uint8_t*>(Q);
    const int lrow = lane >> 2, pch = lane & 3;
    const uint32_t voff = uint32_t(lrow) * uint32_t(ldb) + uint32_t((pch ^ ((lrow >> 2) & 3)) << 4);
    auto issue1 = [&](int ks, int i) __attribute__((always_inline)) {
        uint8_t* sp = smem + (ks % NSTAGE) * SBYTES;
        const uint8_t* g;
        if (i < 2) {
            sp += (wave * 32 + i * 16) * KB;
            g = Pb + int64_t(wave * 32 + i * 16) * ldb;
        } else {
            sp += OPND_BYTES + (wave * QROWS + (i - 2) * 16) * KB;
            g = Qb + int64_t(wave * QROWS + (i - 2) * 16) * ldb;
        }
        __builtin_amdgcn_global_load_lds(g + int64_t(ks) * KB + voff, (lds_void_t*)sp, 16, 0, 0);
    };

    f32x16 acc[MB][NBW];
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    auto rd1 = [&](int ks, int sub, int i, u32x4 (&fa)[MB], u32x4 (&fb)[NBW]) __attribute__((always_inline)) {
        const uint8_t* sp = smem + (ks % NSTAGE) * SBYTES;
        const int chunk = 2 * sub + kg;
        if (i < MB) fa[i] = *reinterpret_cast<const u32x4*>(sp + swz(wm * (MB * 32) + i * 32 + r32, chunk));
        else fb[i - MB] = *reinterpret_cast<const u32x4*>(sp + OPND_BYTES + swz(wn * (NBW * 32) + (i - MB) * 32 + r32, chunk));
    };
    // Explicit per-thread wait for its own loads of the stage being published
    // (the count of its load instructions issued after that stage's last one),
    // then a barrier without __syncthreads()'s release fence, which would
    // drain the loads of later stages too (see gemm_core).
    auto wait_loads = [&](int after) {
        if (after == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        else if (after == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if (after == 7) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
        else if (after == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        else if (after == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        else if (after == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else if (after == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // MF MFMAs on (fa, fb), the NR reads of the next substep one after each of
    // the first MFMAs, and quarter q of the LP loads of pair (ia, ia + 1)
    // spread evenly, in a fixed order (gemm_core's substep).
    auto substep = [&](const u32x4 (&fa)[MB], const u32x4 (&fb)[NBW], bool do_read, int rks, int rsub,
                       u32x4 (&na)[MB], u32x4 (&nb)[NBW], int ia, int q) __attribute__((always_inline)) {
        const int l0 = q * LP / 4, nl = (q + 1) * LP / 4 - l0;
#pragma unroll
        for (int i = 0; i < MF; ++i) {
            Mfma<T>::run(fa[i / NBW], fb[i % NBW], acc[i / NBW][i % NBW]);
            __builtin_amdgcn_sched_barrier(0);
            if (do_read) {
                if (i < NR) rd1(rks, rsub, i, na, nb);
                if (i == MF - 1)
#pragma unroll
                    for (int r = MF; r < NR; ++r) rd1(rks, rsub, r, na, nb);
            }
            if (ia >= 0)
#pragma unroll
                for (int j = 0; j < nl; ++j)
                    if ((j + 1) * MF / nl - 1 == i) {
                        const int l = l0 + j;
                        issue1(ia + (l & 1), l >> 1);
                    }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // The software pipeline of gemm_core: pairs of stages, each pair's loads
    // alternating between its two stages, the pair (ks + 4, ks + 5) loaded
    // into the slots of stages ks - 1 and ks after the barrier of even step ks,
    // spread in quarters over the next four substeps.  Waits: at the barrier
    // of step ks stage ks + 1 must have landed; for even ks the LP loads of
    // the next pair came after its last load, for odd ks one load of its
    // partner and the first half (two quarters) of the next pair.
    constexpr int W_EVEN = LP, W_ODD = 1 + LP / 2, W_FIRST = 1 + LP;
    u32x4 f0a[MB], f0b[NBW], f1a[MB], f1b[NBW];
#pragma unroll
    for (int p = 0; p < 4; p += 2)
#pragma unroll
        for (int l = 0; l < LP; ++l) issue1(p + (l & 1), l >> 1);
    wait_loads(W_FIRST);
    barrier();
#pragma unroll
    for (int i = 0; i < NR; ++i) rd1(0, 0, i, f0a, f0b);
    __builtin_amdgcn_sched_barrier(0);

    auto step = [&](int ks, int after, int pa, int qa, int pb, int qb) __attribute__((always_inline)) {
        substep(f0a, f0b, true, ks, 1, f1a, f1b, pa, qa);
        wait_loads(after);
        barrier();     // stage ks+1 visible everywhere; every read of stage ks done
        __builtin_amdgcn_sched_barrier(0);
        substep(f1a, f1b, true, ks + 1, 0, f0a, f0b, pb, qb);
    };
    step(0, W_EVEN, -1, 0, 4, 0);
    step(1, W_ODD, 4, 1, 4, 2);
    int ks = 2;
    for (; ks + 6 <= nk; ks += 2) {
        step(ks, W_EVEN, ks + 2, 3, ks + 4, 0);
        step(ks + 1, W_ODD, ks + 4, 1, ks + 4, 2);
    }
    step(ks, W_EVEN, ks + 2, 3, -1, 0);
    step(ks + 1, 1, -1, 0, -1, 0);
    step(ks + 2, 0, -1, 0, -1, 0);
    substep(f0a, f0b, true, nk - 1, 1, f1a, f1b, -1, 0);
    substep(f1a, f1b, false, 0, 0, f0a, f0b, -1, 0);
    __syncthreads();   // every wave is done with the operand stages

    const Ep ep = make_ep();
    const bool off_diag = ti != tj * TN / GT;
    const EpiPasses ps = ep.passes(off_diag);
    const bool run_b = ps.run_b, write_b = ps.write_b, run_a = ps.run_a, hand_over = ps.hand_over;
    constexpr int WC = NBW * 32;                         // columns of a wave's sub-tile
    constexpr int NT = 2 * NBW;                          // epilogue tasks per lane and pass
    const int64_t gi_w = int64_t(ti) * GT + wm * (MB * 32);
    const int64_t gj_w = int64_t(tj) * TN + wn * WC;
    uint8_t* st = smem + wave * (32 * WC * 4);           // 32 rows x WC columns of fp32

    // One 32-row block of the wave's sub-tile (gemm_core's round, without the
    // captured operand).
    auto round = [&](const int a, const f32x16 (&ac)[NBW]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v4 = {ac[b][4 * g], ac[b][4 * g + 1], ac[b][4 * g + 2], ac[b][4 * g + 3]};
                *reinterpret_cast<f32x4*>(st + st_off(b * 32 + r32, g * 8 + kg * 4)) = v4;
            }
        __builtin_amdgcn_wave_barrier();
        if (run_b) {
            // mirrored pass: column j of the sub-tile, rows 8 ic .. 8 ic + 7
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int j = (lane >> 2) + 16 * t, ic = lane & 3;
                f32x4* s0 = reinterpret_cast<f32x4*>(st + st_off(j, ic * 8));
                f32x4* s1 = reinterpret_cast<f32x4*>(st + st_off(j, ic * 8 + 4));
                const f32x4 lo = *s0, hi = *s1;
                f32x8 v, o;
#pragma unroll
                for (int e = 0; e < 4; ++e) { v.v[e] = lo[e]; v.v[4 + e] = hi[e]; }
                const int64_t oj = gj_w + j, oi = gi_w + a * 32 + ic * 8;
                ep.operand(oj, oi, o);
                ep.combine(oj, oi, v, o);
                if (write_b) ep.mirror(oj, oi, v);
                if (hand_over) {
                    *s0 = f32x4{v.v[0], v.v[1], v.v[2], v.v[3]};
                    *s1 = f32x4{v.v[4], v.v[5], v.v[6], v.v[7]};
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (run_a) {
            // tile pass: row of the sub-tile, columns 8 cc .. 8 cc + 7 (4 NBW lanes per row)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int cc = lane % (4 * NBW), row = lane / (4 * NBW) + (16 / NBW) * t;
                f32x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v.v[e] = *reinterpret_cast<const float*>(st + st_off(cc * 8 + e, row));
                if (!hand_over) ep.tile_value(v);
                ep.tile(gi_w + a * 32 + row, gj_w + cc * 8, v);
            }
            __builtin_amdgcn_wave_barrier();
        }
    };
    round(0, acc[0]);
    round(1, acc[1]);
    if constexpr (MB == 4) {
        round(2, acc[2]);
        round(3, acc[3]);
    }
}

}  // namespace mo_gemm

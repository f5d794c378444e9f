// The tiled NT GEMM on MFMA shared by the Muon and Shampoo kernels: the K
// pipeline through LDS and the two-pass epilogue driver.  The operands and what
// happens to the results are the caller's: it passes the operand rows and an
// epilogue object.
#pragma once

#include "device_common.h"

namespace mo_gemm {

// ============================================================================
// NT GEMM family on MFMA:  C[i][j] = sum_k P[i][k] * Q[j][k]
// ============================================================================
//
// Workgroup tile 256 x 256, 256 threads = 4 wavefronts in a 2 x 2 grid; each
// wavefront owns a 128 x 128 sub-tile = 4 x 4 MFMA blocks of 32 x 32 (256 fp32
// accumulators per lane, held in AGPRs).  Per K stage every operand row
// contributes 64 bytes (32 bf16 / 16 fp32): 2 x 256 rows x 64 B = 32 KB, in a
// ring of five stages in LDS (all 160 KB of the CU's LDS, one workgroup per
// CU).  Global data goes straight to LDS (global_load_lds_dwordx4, no VGPR
// round trip), two stages at a time, spread between the MFMAs (see the main
// loop below).
//
// A direct-to-LDS load writes lane l's 16 bytes at (wave base + 16 l), so each
// lane fetches the global chunk that belongs at its physical (swizzled) slot.
//
// MFMA operands.  bf16: v_mfma_f32_32x32x16_bf16 takes 8 consecutive k per
// lane; lane l supplies row (l % 32) and k-group (l / 32).  fp32:
// v_mfma_f32_32x32x2_f32 takes one k per lane; a 16-byte chunk of 4 floats feeds
// four of them.  A and B fragments use the same lane -> k assignment, so the
// sum over all k is exact regardless of how k is split among lanes.  The 32 x 32
// result sits in lane l, register v at row (v/4)*8 + (l/32)*4 + v%4, col l%32.
//
// Epilogue, per wavefront and per 32-row block of its sub-tile: the fp32
// values are staged by column in a private 16 KB LDS slice, then written out
// as 16-byte chunks in the mirrored orientation (pass B, where the transposed
// product is needed; it also forms the final values) and in the tile's own
// orientation (pass A: 16 lanes cover one 128-column row).  What the passes
// compute and where they write is the caller's epilogue object (below).

constexpr int GT = MO_GEMM_TILE;           // 256
constexpr int G_THREADS = 256;
constexpr int KB = 64;                     // bytes of K per LDS stage and row
constexpr int NSTAGE = 5;                  // LDS ring depth
constexpr int OPND_BYTES = GT * KB;        // 16 KB per operand per stage
constexpr int GEMM_LDS = NSTAGE * 2 * OPND_BYTES;  // 160 KB at full width, all of the CU's LDS

typedef __attribute__((address_space(3))) void lds_void_t;

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    static MO_DEV void run(const u32x4& a, const u32x4& b, f32x16& acc) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static MO_DEV void run(const u32x4& a, const u32x4& b, f32x16& acc) {
        const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
    }
};

// 64-byte rows of four 16-byte chunks; logical chunk c of row r sits at
// c ^ ((r >> 2) & 3).  The LDS serves 16 lanes x 16 bytes per clock from 64
// banks; 16 consecutive rows read at one logical chunk then fall on 16
// distinct 16-byte bank groups (four rows per 256-byte bank line, each at a
// different chunk).
MO_DEV int swz(int row, int chunk) { return row * KB + ((chunk ^ ((row >> 2) & 3)) << 4); }

// Staging slice of one wave (16 KB): the fp32 results of one 32-row block of
// its 128 x 128 sub-tile, stored by column.  Value (column j, row i) sits in
// the 256-byte line j / 2, in 16-byte group G (rows i & ~3 .. + 3 of the
// column); G XORs the group's position in the line with bits of j so that
// the three access patterns (16-byte accumulator writes of 16 consecutive
// columns, 16-byte reads of 4 columns x 4 row groups, and 4-byte reads of 16
// columns 8 apart x 4 rows) each hit distinct banks.
MO_DEV int st_off(int j, int i) {
    const int p = j >> 1;
    const int g = ((j & 1) | ((i >> 2) << 1)) ^ (((p & 7) << 1) ^ ((p >> 3) & 7));
    return p * 256 + g * 16 + (i & 3) * 4;
}

// Which epilogue passes run on a tile (see gemm_core).
struct EpiPasses {
    bool run_b;       // mirrored pass runs (reads the staged values by column)
    bool write_b;     // ... and writes them at the mirrored position
    bool run_a;       // tile pass runs
    bool hand_over;   // the mirrored pass forms the final values and hands them to the tile pass
};

// One 256 x TN tile of C = P Q^T, TN = 64 NB (NB = 4: the full 256 x 256 tile; 2 and 1:
// the half and quarter widths the host uses where full tiles would leave CUs
// idle).  Each wavefront owns 128 x (TN / 2) = 4 x NB blocks of 32 x 32.  A
// narrower tile accumulates every output element over the same K in the same
// order, so its results are bit-identical to the full tile's.
//
// Pm and Qm are the operand matrices (row stride ld elements, a multiple of
// 256; ld is also the K extent); the tile takes P rows 256 ti .. + 255 and Q
// rows TN tj .. + TN - 1.  make_ep() returns the epilogue object, which supplies
//   CAP                      (bf16 only) capture the epilogue operand from the
//                            Q stage at K block ti instead of reading it
//   KROT                     start the K loop at stage krot instead of 0 (not
//                            with CAP)
//   passes(off_diag)         which passes run (EpiPasses)
//   operand(oj, oi, o)       the mirrored pass's epilogue operand at (oj, oi..+7)
//   combine(oj, oi, v, o)    final values of the mirrored pass at (oj, oi..+7)
//   mirror(oj, oi, v)        write them at row oj, columns oi .. oi + 7
//   tile_value(v)            final values in the tile pass when nothing is handed over
//   tile(gi, gj, v)          write row gi, columns gj .. gj + 7
template <typename T, int NB, class MakeEp>
__device__ __forceinline__ void gemm_core(uint8_t* smem, const T* Pm, const T* Qm, int64_t ld, int ti,
                                          int tj, const MakeEp& make_ep, int krot = 0) {
    using Ep = decltype(make_ep());
    constexpr int TN = 64 * NB;                  // tile columns = rows of Q
    constexpr int SBYTES = OPND_BYTES + TN * KB; // one stage: P (256 rows) then Q (TN rows)
    constexpr int LS = 4 + NB;                   // load instructions per stage and wave
    constexpr int LP = 2 * LS;                   // ... per pair of stages
    constexpr int MF = 4 * NB;                   // MFMA blocks per wave and substep
    constexpr int NR = 4 + NB;                   // fragment reads per substep
    // operand rows of this tile: P rows 256 ti .., Q rows TN tj .. (row stride ld)
    const T* P = Pm + int64_t(ti) * GT * ld;
    const T* Q = Qm + int64_t(tj) * TN * ld;
    const int64_t ldb = ld * int64_t(sizeof(T));             // row stride in bytes
    const int nk = int(ldb / KB);                              // K stages
    // Logical stage ks reads K stage (ks + krot) mod nk when the epilogue asks
    // for a rotated K order (Ep::KROT); each output is still one sequential
    // sum over all of K, only its starting point moves.
    auto kstage = [&](int ks) __attribute__((always_inline)) {
        if constexpr (Ep::KROT) {
            const int p = ks + krot;
            return p >= nk ? p - nk : p;
        } else {
            return ks;
        }
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, kg = lane >> 5;

    // direct-to-LDS loads: wave w fills rows [64 w, 64 w + 64) of P and rows
    // [TN/4 w, TN/4 (w + 1)) of Q, 16 rows (1 KB) per instruction; lane l ->
    // row + l/4, physical chunk l%4.  The rows of one instruction start at a
    // wave-uniform address (SGPRs); the lane's part, the same for every
    // instruction since the swizzle depends on the row modulo 16 only, is one
    // 32-bit offset (16 rows of at most 32 MB).
    const uint8_t* Pb = reinterpret_cast<const uint8_t*>(P);
    const uint8_t* Qb = reinterpret_cast<const uint8_t*>(Q);
    const int lrow = lane >> 2, pch = lane & 3;
    const uint32_t voff = uint32_t(lrow) * uint32_t(ldb) + uint32_t((pch ^ ((lrow >> 2) & 3)) << 4);
    // Load instruction i (0 .. LS-1) of stage ks: P rows 64 wave + 16 i (i < 4),
    // else Q rows TN/4 wave + 16 (i - 4).
    auto issue1 = [&](int ks, int i) __attribute__((always_inline)) {
        uint8_t* sp = smem + (ks % NSTAGE) * SBYTES;
        const uint8_t* g;
        if (i < 4) {
            sp += (wave * 64 + i * 16) * KB;
            g = Pb + int64_t(wave * 64 + i * 16) * ldb;
        } else {
            sp += OPND_BYTES + (wave * (TN / 4) + (i - 4) * 16) * KB;
            g = Qb + int64_t(wave * (TN / 4) + (i - 4) * 16) * ldb;
        }
        __builtin_amdgcn_global_load_lds(g + int64_t(kstage(ks)) * KB + voff, (lds_void_t*)sp, 16, 0, 0);
    };

    f32x16 acc[4][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    // Fragment i of one 16-deep K substep: A chunk i (i < 4) or B chunk i - 4.
    auto rd1 = [&](int ks, int sub, int i, u32x4 (&fa)[4], u32x4 (&fb)[NB]) __attribute__((always_inline)) {
        const uint8_t* sp = smem + (ks % NSTAGE) * SBYTES;
        const int chunk = 2 * sub + kg;
        if (i < 4) fa[i] = *reinterpret_cast<const u32x4*>(sp + swz(wm * 128 + i * 32 + r32, chunk));
        else fb[i - 4] = *reinterpret_cast<const u32x4*>(sp + OPND_BYTES + swz(wn * (TN / 2) + (i - 4) * 32 + r32, chunk));
    };
    // Workgroup barrier without the release fence of __syncthreads(), which
    // would also drain the direct-to-LDS loads still in flight for later
    // stages.  Each thread first waits for its own loads of the stage being
    // published (explicit vmcnt: the number of its load instructions issued
    // after that stage's last one) and for its LDS reads (lgkmcnt).
    auto wait_loads = [&](int after) {
        if (after == 17) asm volatile("s_waitcnt vmcnt(17)" ::: "memory");
        else if (after == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (after == 13) asm volatile("s_waitcnt vmcnt(13)" ::: "memory");
        else if (after == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        else if (after == 11) asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
        else if (after == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        else if (after == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        else if (after == 7) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
        else if (after == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        else if (after == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // lgkmcnt(0) through the builtin (gfx9 encoding: vmcnt and expcnt at their
    // maxima), so the compiler knows every fragment read has landed and adds
    // no wait of its own after the barrier.
    auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // The MF MFMAs of one substep on (fa, fb).  The NR fragment reads of the
    // next substep (stage rks, substep rsub, into na / nb) follow the first
    // MFMAs, one each (the surplus after the last when NR > MF).  When ia >= 0,
    // quarter q of the LP loads of the pair (ia, ia + 1) is spread evenly over
    // the MFMAs, load l being instruction l / 2 of stage ia + (l & 1).  The
    // order is fixed (sched_barrier), so reads and loads stream out between
    // the MFMAs instead of in bursts that would stall instruction issue behind
    // a full load queue.
    auto substep = [&](const u32x4 (&fa)[4], const u32x4 (&fb)[NB], bool do_read, int rks, int rsub,
                       u32x4 (&na)[4], u32x4 (&nb)[NB], int ia, int q) __attribute__((always_inline)) {
        const int l0 = q * LP / 4, nl = (q + 1) * LP / 4 - l0;
#pragma unroll
        for (int i = 0; i < MF; ++i) {
            Mfma<T>::run(fa[i / NB], fb[i % NB], acc[i / NB][i % NB]);
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

    // Software pipeline over K (nk >= 8 and even: every padded dimension is a
    // multiple of 256).  Stage s occupies ring slot s % NSTAGE.  Entering step
    // ks, F0 holds the fragments of (ks, substep 0).  The barrier sits between
    // the two substeps, so the MFMAs after it use fragments already in
    // registers while the reads for the next stage land.
    //
    // Stages are loaded in pairs (2p, 2p + 1), whose 64-byte row pieces are
    // the two halves of the same 128-byte lines, with the two stages'
    // instructions alternating so both halves of a line are requested back to
    // back.  The pair (ks + 4, ks + 5) goes into the slots of stages ks - 1 and
    // ks, which every wave has finished reading once the barrier of even step
    // ks has passed; its LP loads are spread in quarters over the four
    // substeps that follow (second of step ks, both of ks + 1, first of
    // ks + 2).  At the barrier of step ks, stage ks + 1 must have landed: for
    // even ks it is the second of its pair and all LP loads of the next pair
    // came after it; for odd ks it is the first of its pair, followed by one
    // load of its partner and the first half of the next pair.
    constexpr int W_EVEN = LP, W_ODD = 1 + LP / 2, W_FIRST = 1 + LP;
    u32x4 f0a[4], f0b[NB], f1a[4], f1b[NB];
#pragma unroll
    for (int p = 0; p < 4; p += 2)
#pragma unroll
        for (int l = 0; l < LP; ++l) issue1(p + (l & 1), l >> 1);
    wait_loads(W_FIRST);
    barrier();
#pragma unroll
    for (int i = 0; i < NR; ++i) rd1(0, 0, i, f0a, f0b);
    __builtin_amdgcn_sched_barrier(0);
    // Epilogue operand capture (Ep::CAP, bf16 operands): for epilogues whose
    // operand at (i, j) is Q[j][i], the value sits in the Q stage that holds
    // K columns 256 ti + 128 wm .. of row j.  K stage 8 ti + 4 wm + r covers rows
    // 32 r .. 32 r + 31 of this wave's sub-tile, so while that stage is in LDS
    // each lane copies the 2 NB chunks its mirrored-pass tasks of round r need
    // (task t: column j = lane / 4 + 16 t, rows 8 (lane % 4) .. + 7) into
    // registers, and the epilogue reads nothing from global memory.
    constexpr bool CAP = Ep::CAP;
    constexpr int NT = 2 * NB;                           // epilogue tasks per lane and pass
    const int64_t gi_w = int64_t(ti) * GT + wm * 128;   // this wave's sub-tile origin
    const int64_t gj_w = int64_t(tj) * TN + wn * (TN / 2);
    u32x4 pre[CAP ? 4 : 1][NT];
    const int cap0 = ti * (GT * int(sizeof(T)) / KB) + wm * 4;
    auto capture = [&](int ks) __attribute__((always_inline)) {
        if constexpr (CAP) {
            const int r = ks - cap0;   // wave-uniform
            if (r >= 0 && r < 4) {
                // Register selects rather than pre[r][t] = ..., which would
                // index the array dynamically and move it to scratch memory.
                const uint8_t* sq = smem + (ks % NSTAGE) * SBYTES + OPND_BYTES;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const u32x4 c = *reinterpret_cast<const u32x4*>(
                        sq + swz(wn * (TN / 2) + (lane >> 2) + 16 * t, lane & 3));
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) pre[rr][t] = r == rr ? c : pre[rr][t];
                }
            }
        }
    };

    // (pa, qa): pair and quarter of loads issued in this step's first
    // substep; (pb, qb) in its second (pair -1: none).
    auto step = [&](int ks, int after, int pa, int qa, int pb, int qb) __attribute__((always_inline)) {
        substep(f0a, f0b, true, ks, 1, f1a, f1b, pa, qa);
        capture(ks);   // stage ks is still resident until the barrier below
        wait_loads(after);
        barrier();     // stage ks+1 visible everywhere; every read of stage ks done
        __builtin_amdgcn_sched_barrier(0);
        substep(f1a, f1b, true, ks + 1, 0, f0a, f0b, pb, qb);
    };
    // the prologue issued pairs (0, 1) and (2, 3) whole
    step(0, W_EVEN, -1, 0, 4, 0);
    step(1, W_ODD, 4, 1, 4, 2);
    int ks = 2;
    for (; ks + 6 <= nk; ks += 2) {
        step(ks, W_EVEN, ks + 2, 3, ks + 4, 0);
        step(ks + 1, W_ODD, ks + 4, 1, ks + 4, 2);
    }
    // ks == nk - 4: the last pair (nk - 2, nk - 1) lacks its last quarter
    step(ks, W_EVEN, ks + 2, 3, -1, 0);
    step(ks + 1, 1, -1, 0, -1, 0);
    step(ks + 2, 0, -1, 0, -1, 0);
    substep(f0a, f0b, true, nk - 1, 1, f1a, f1b, -1, 0);
    capture(nk - 1);
    substep(f1a, f1b, false, 0, 0, f0a, f0b, -1, 0);
    __syncthreads();   // every wave is done with the operand stages

    // The epilogue object is made only now, so nothing it loads is held in
    // registers through the main loop.
    const Ep ep = make_ep();
    // Which passes run and write is the epilogue's choice, given whether the
    // tile straddles the diagonal of a square product.
    const bool off_diag = ti != tj * TN / GT;
    const EpiPasses ps = ep.passes(off_diag);
    const bool run_b = ps.run_b, write_b = ps.write_b, run_a = ps.run_a, hand_over = ps.hand_over;

    uint8_t* st = smem + wave * (32 * (TN / 2) * 4);   // 32 rows x TN/2 columns of fp32
    // One 32-row block of the wave's sub-tile; called with literal indices so
    // the accumulator and capture arrays are never indexed dynamically.
    auto round = [&](const int a, const f32x16 (&ac)[NB], const u32x4 (&pf)[NT]) __attribute__((always_inline)) {
        // accumulators: lane holds column 32 b + lane % 32, rows 8 g + 4 (lane / 32) .. + 3
#pragma unroll
        for (int b = 0; b < NB; ++b)
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
                if constexpr (CAP) {
                    const bf16x8 raw = __builtin_bit_cast(bf16x8, pf[t]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o.v[e] = (float)raw[e];
                } else {
                    ep.operand(oj, oi, o);
                }
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
            // tile pass: row of the sub-tile, columns 8 cc .. 8 cc + 7 (4 NB lanes per row)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int cc = lane % (4 * NB), row = lane / (4 * NB) + (16 / NB) * t;
                f32x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v.v[e] = *reinterpret_cast<const float*>(st + st_off(cc * 8 + e, row));
                if (!hand_over) ep.tile_value(v);
                ep.tile(gi_w + a * 32 + row, gj_w + cc * 8, v);
            }
            __builtin_amdgcn_wave_barrier();
        }
    };
    round(0, acc[0], pre[0]);
    round(1, acc[1], pre[CAP ? 1 : 0]);
    round(2, acc[2], pre[CAP ? 2 : 0]);
    round(3, acc[3], pre[CAP ? 3 : 0]);
}


}  // namespace mo_gemm

// producers.hip -- LayerNorm / adaptive-LayerNorm -> FP8 producers for gfx950.
//
// What is computed (per row of a bf16 (rows, dim) activation) follows the
// "adaptive-layernorm-producers" README ("Available Functions", "Tensor
// Contract"): LayerNorm without affine weights, DiT modulation
// (xhat * (1 + scale)) + shift (operation order from the h3-blackwell-runtime
// page, "NVFP4 Modulation Producer Fusion", "Exactness Contract"), then
// static-scale e4m3 or block-16 e2m1 quantization.  The same row kernels
// also write the MX block formats (E8M0 scale per 32 elements, OCP MX v1.0),
// and a sibling kernel computes RMSNorm with segment-selected modulation in
// bf16 operations (RL-Kernel norm_modulate page; h3 page, "Implementation
// Phases").
//
// This file: the FP8 producers (static scale and MXFP8) for every operand
// form, their fallbacks and launchers, and the standalone quantizer.  The
// FP4 producers live in fp4.hip, the RMSNorm producer in rmsmod.hip, the
// shared row machinery in rows.hpp.
#include "rows.hpp"
#include "timeline.hpp"

// Where a row kernel issues the loads of its streamed operands (per-token
// scale / shift rows, temb chunks), relative to the row statistics.
enum LoadPoint : int {
    kWithX = 0,        // with the row's x
    kAfterMean = 1,    // after the mean (first reduction)
    kAfterRstd = 2,    // after rstd (second reduction)
};

namespace alnp {

// MX: MXFP8 output, one E8M0 scale per 32 elements (the four vectors of a
// lane quad) in place of the static act_scale.  FULL: the row fills every
// vector slot (dim / 8 == VPT * WAVES * 64, as for dim 2048 and 3072), so the
// last slot needs no bounds check, zero fill or predicated stores; the
// launcher picks it, and the arithmetic is the same.
template <int VPT, int WAVES, int FORM, bool MX = false, bool FULL = false, bool PRE = false,
          bool PAIRS = false>
__global__ __launch_bounds__(WAVES * 64) void k_adaln_fp8_rows(Fp8Args a)
{
    __shared__ float red[32];  // two sets of per-wave partials
    constexpr int T = WAVES * 64;
    // Register arrays per operand kind (size 1 where the form has none).
    constexpr bool kBf16Ops = FORM == kBcast || FORM == kPtok || FORM == kTable || FORM == kAwq;
    constexpr int NB = kBf16Ops ? VPT : 1;
    // Table rows are held from the start for up to 4 vectors per thread; with
    // more, holding them (16 floats per vector) would spill, so each vector's
    // table values are read in the output pass instead.
    constexpr bool kTableEarly = FORM == kTable && VPT <= 4;
    constexpr int NT = kTableEarly ? 2 * VPT : 1;
    constexpr int N8 = FORM == kModFp8 ? VPT : 1;
    constexpr int NI = FORM == kAwq ? VPT : 1;
    // PRE: shared operands formed ahead of the row (see below), for up to
    // three vectors per thread, so that the extra 16 or 24 registers per
    // vector leave every row of the large calls resident.
    constexpr bool kPre = PRE && (FORM == kBcast || FORM == kModFp8 || FORM == kAwq) && VPT <= 3;
    constexpr int NP = kPre ? VPT : 1;
    const int t = threadIdx.x;
    const int dim = a.dim;
    const int nvec = dim >> 3;
    const float inv = MX ? 0.f : 1.0f / *a.act_scale;
    const int64_t row = grid_row();
    if (row >= a.rows)
        return;  // whole workgroup
    ALNP_TL_VARS;
    ALNP_TL_MARK(0);
    {
        // Modulation operands shared by every row ((dim,) vectors, kept in
        // cache) are requested before x.  With kPre the broadcast, modfp8
        // and AWQ forms turn them into (1 + scale) and shift while x is in
        // flight: they land first (L2 hits), and the output pass after the
        // row's last bytes arrive is two to four operations per element
        // shorter.  2520 x 3072 cold: modfp8 7.01 -> 6.77 us, AWQ 7.45 ->
        // 7.33 us (A-B, same box, bit-identical).  Streamed per-row operands
        // (load_streamed below) are requested after the row statistics.
        // With kPre, the operands that only the output pass reads (the
        // broadcast shift, AWQ's inv_s) are requested after the mean
        // instead: every load a CU issues ahead of x holds up the x of its
        // later rows, and these arrive while the variance is summed.
        // Broadcast 6.88 -> 6.74 us, AWQ 7.35 -> 7.18 us (A-B, bit-identical;
        // AWQ's shift and the modfp8 shift measured slower that way).  The
        // MXFP8 forms, not measured so, keep every operand ahead of x.
        constexpr bool kLateShift = kPre && !MX && FORM == kBcast;
        constexpr bool kLateInvS = kPre && !MX && FORM == kAwq;
        uint4 scv[NB], shv[NB];
        uint2 sc8[N8], sh8[N8];
        uint4 isv[NI];
        if (FORM == kBcast || FORM == kAwq) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                scv[v] = ld_row<false>(a.scale, v * T + t, nvec, !FULL && v == VPT - 1);
                if (!kLateShift)
                    shv[v] = ld_row<false>(a.shift, v * T + t, nvec, !FULL && v == VPT - 1);
                if (FORM == kAwq && !kLateInvS)
                    isv[v] = ld_row<false>(a.inv_s, v * T + t, nvec, !FULL && v == VPT - 1);
            }
        } else if (FORM == kModFp8) {
            // PAIRS (kPre FP8 rows that fill every slot, operands 16-byte
            // aligned; the launcher checks): lane pairs halve the load
            // instructions issued ahead of x.  The even lane loads 16 scale
            // bytes and the odd lane 16 shift bytes for the pair's two
            // vectors (8 * (i & ~1), inside the row since the slot count is
            // even), and each passes the other the half it needs.  2520 x
            // 3072 cold 6.76 -> 6.67 us (A-B, bit-identical); as a run-time
            // branch in one kernel 6.95, and in the FP4 kernel slower.
            constexpr bool kPairs = PAIRS && kPre && FULL && !MX;
            if (kPairs) {
                const bool odd = t & 1;
                const uint8_t* src = odd ? a.shift_fp8 : a.scale_fp8;
#pragma unroll
                for (int v = 0; v < VPT; ++v) {
                    const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * ((v * T + t) & ~1));
                    const uint32_t s0 = odd ? w.x : w.z, s1 = odd ? w.y : w.w;
                    const uint32_t r0 = __builtin_amdgcn_mov_dpp(s0, 0xB1, 0xF, 0xF, false);  // lane ^ 1
                    const uint32_t r1 = __builtin_amdgcn_mov_dpp(s1, 0xB1, 0xF, 0xF, false);
                    sc8[v] = odd ? make_uint2(r0, r1) : make_uint2(w.x, w.y);
                    sh8[v] = odd ? make_uint2(w.z, w.w) : make_uint2(r0, r1);
                }
            } else {
#pragma unroll
                for (int v = 0; v < VPT; ++v) {
                    sc8[v] = ld_fp8x8(a.scale_fp8, v * T + t, nvec, !FULL && v == VPT - 1);
                    sh8[v] = ld_fp8x8(a.shift_fp8, v * T + t, nvec, !FULL && v == VPT - 1);
                }
            }
        }
        uint4 xv[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            xv[v] = ld_row<true>(a.x + row * dim, v * T + t, nvec, !FULL && v == VPT - 1);
        ALNP_TL_MARK(1);
        const float sdeq = FORM == kModFp8 ? *a.scale_deq : 0.f;
        const float hdeq = FORM == kModFp8 ? *a.shift_deq : 0.f;
        // tp = 1 + scale, hp = shift (fp32, the same roundings as in the
        // output pass); AWQ keeps its shift packed (registers).
        float tp[NP][8], hp[NP][8];
        if (kPre) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                float sc[8], sh[8];
                if (FORM == kModFp8) {
                    unpack_e4m3x8(sc8[v], sc);
                    unpack_e4m3x8(sh8[v], sh);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sc[e] = sc[e] * sdeq;
                        sh[e] = sh[e] * hdeq;
                    }
                } else {
                    unpack8(scv[v], sc);
                    if (!kLateShift)
                        unpack8(shv[v], sh);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    tp[v][e] = 1.0f + sc[e];
                    hp[v][e] = kLateShift ? 0.f : sh[e];
                }
                // Keep the compiler from sinking this into the output pass.
                asm volatile("" : "+v"(tp[v][0]), "+v"(tp[v][1]), "+v"(tp[v][2]), "+v"(tp[v][3]),
                                  "+v"(tp[v][4]), "+v"(tp[v][5]), "+v"(tp[v][6]), "+v"(tp[v][7]));
                if (FORM != kAwq && !kLateShift)
                    asm volatile("" : "+v"(hp[v][0]), "+v"(hp[v][1]), "+v"(hp[v][2]), "+v"(hp[v][3]),
                                      "+v"(hp[v][4]), "+v"(hp[v][5]), "+v"(hp[v][6]), "+v"(hp[v][7]));
            }
        }
        // Table rows (fp32, shared by every row, L2-resident): also requested
        // before the reductions so their latency is not added at the end.
        float4 tsv[NT], thv[NT];
        if (kTableEarly) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int i = v * T + t;
                const int j = i < nvec ? 8 * i : 0;
                const float4* ts = reinterpret_cast<const float4*>(a.table + (int64_t)a.scale_idx * dim + j);
                const float4* th = reinterpret_cast<const float4*>(a.table + (int64_t)a.shift_idx * dim + j);
                tsv[2 * v] = ts[0];
                tsv[2 * v + 1] = ts[1];
                thv[2 * v] = th[0];
                thv[2 * v + 1] = th[1];
            }
        }

        // Per-token rows and temb chunks, streamed, are requested only once
        // rstd is known.  Every row is resident from the start and every
        // wave's x is requested at once, so the last waves receive their
        // data near the end of the stream and then run all their
        // arithmetic: that serial tail is what separates the kernel from a
        // memory-only pass over the same bytes.  With the operands
        // requested after the statistics, each wave's bytes arrive in two
        // phases: the statistics run while the operands are in flight
        // behind other waves' traffic, and only the output pass remains
        // after the last bytes land.  Per-token 2520 x 3072: 10.80 -> 10.18
        // us cold (A-B, same box; after the mean: 10.27), bit-identical.
        constexpr int kLoad = kAfterRstd;
        auto load_streamed = [&](int when) {
            if ((FORM == kPtok || FORM == kTable) && when == kLoad) {
                const uint16_t* scr = FORM == kPtok ? a.scale + row * dim
                                                    : a.temb + (row * a.chunks + a.scale_idx) * dim;
                const uint16_t* shr = FORM == kPtok ? a.shift + row * dim
                                                    : a.temb + (row * a.chunks + a.shift_idx) * dim;
#pragma unroll
                for (int v = 0; v < VPT; ++v) {
                    scv[v] = ld_row<true>(scr, v * T + t, nvec, !FULL && v == VPT - 1);
                    shv[v] = ld_row<true>(shr, v * T + t, nvec, !FULL && v == VPT - 1);
                }
            }
        };
        load_streamed(kWithX);
        const bool tail_ok = FULL || (VPT - 1) * T + t < nvec;
        auto reduce = [&](float v, int k) { return group_sum(v, red + 16 * k, WAVES); };
        float d[VPT][8];
        const float xsum = thread_sum<VPT>(xv);
        ALNP_TL_MARK_AFTER(2, xsum);
        const float mean = reduce(xsum, 0) * a.inv_dim;
        load_streamed(kAfterMean);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            if (kLateShift)
                shv[v] = ld_row<false>(a.shift, v * T + t, nvec, !FULL && v == VPT - 1);
            if (kLateInvS)
                isv[v] = ld_row<false>(a.inv_s, v * T + t, nvec, !FULL && v == VPT - 1);
        }
        const float rstd = row_rstd<VPT>(xv, tail_ok, mean, a.inv_dim, a.eps, reduce, d);
        ALNP_TL_MARK_AFTER(3, rstd);
        load_streamed(kAfterRstd);

#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int i = v * T + t;
            if (v == VPT - 1 && !tail_ok)
                continue;
            float sc[8], sh[8];
            if (FORM == kNone || kPre) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sc[e] = 0.f;
                    sh[e] = 0.f;
                }
                if (kLateShift)
                    unpack8(shv[v], sh);
            } else if (FORM == kModFp8) {
                // Dequantize: e4m3 value times its fp32 scalar, one rounding.
                unpack_e4m3x8(sc8[v], sc);
                unpack_e4m3x8(sh8[v], sh);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sc[e] = sc[e] * sdeq;
                    sh[e] = sh[e] * hdeq;
                }
            } else {
                unpack8(scv[v], sc);
                unpack8(shv[v], sh);
                if (FORM == kTable) {
                    float4 t0, t1, h0, h1;
                    if (kTableEarly) {
                        t0 = tsv[2 * v];
                        t1 = tsv[2 * v + 1];
                        h0 = thv[2 * v];
                        h1 = thv[2 * v + 1];
                    } else {
                        const float4* ts = reinterpret_cast<const float4*>(a.table + (int64_t)a.scale_idx * dim + 8 * i);
                        const float4* th = reinterpret_cast<const float4*>(a.table + (int64_t)a.shift_idx * dim + 8 * i);
                        t0 = ts[0];
                        t1 = ts[1];
                        h0 = th[0];
                        h1 = th[1];
                    }
                    const float ts[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
                    const float th[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sc[e] = sc[e] + ts[e];
                        sh[e] = sh[e] + th[e];
                    }
                }
            }
            float is[8];
            if (FORM == kAwq)
                unpack8(isv[v], is);
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xhat = d[v][e] * rstd;
                float y = kPre ? (xhat * tp[v][e]) + (kLateShift ? sh[e] : hp[v][e])
                               : (xhat * (1.0f + sc[e])) + sh[e];
                if (FORM == kAwq)
                    y = y * is[e];  // per-channel smoothing before the static scale
                q[e] = MX ? y : y * inv;
            }
            if (!MX)
                sat448x8(q);
            if (MX) {
                // Block scale 2^E from the quad's maximum; elements y * 2^-E
                // (exact), saturated at 448.  The quad's lanes store the same
                // scale byte.
                const int E = mx_scale_exp(quad_max(absmax8(q)), 8);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    q[e] = sat448(__builtin_amdgcn_ldexpf(q[e], -E));
                a.mx_scales[row * (dim >> 5) + (i >> 2)] = (uint8_t)(E + 127);
            }
            st_stream(a.out + row * dim + (int64_t)i * 8,
                      make_uint2(pack_e4m3x4(q[0], q[1], q[2], q[3]),
                                 pack_e4m3x4(q[4], q[5], q[6], q[7])));
        }
        if (t == 0) {
            if (a.row_mean) a.row_mean[row] = mean;
            if (a.row_rstd) a.row_rstd[row] = rstd;
        }
        ALNP_TL_MARK(4);
        ALNP_TL_RECORD(row, WAVES);
    }
}

// Table form with the two selected fp32 table rows staged in LDS and shared by
// the two rows of a workgroup.  Holding the table in registers costs ~50
// VGPRs per thread, which leaves room for only 2048 of the 2520 rows of the
// Wan workload on the chip at once; from LDS the kernel keeps the per-token
// kernel's register budget and reads each table element from L2 once per
// two rows instead of once per row.  When the table loads (L2 hits) are
// issued is set per output format below.
constexpr int kTableRows = 2;     // rows per workgroup
// LDS bound: 2 table rows * 8192 * 4 B = 64 KiB.  The row shapes of at most
// four waves, which this kernel takes, end at dim 7168 (57344 bytes) anyway.
constexpr int kTableMaxDim = 8192;
// Up to this many rows the table form runs the rows kernel instead, which
// holds each thread's table values in registers: with few rows resident,
// registers are not what limits the kernel, and skipping the LDS staging and
// its barrier shortens the call (51 x 1536: 3.28 -> 2.31 us; 256 x 3072:
// 3.48 -> 2.72 us; even at 512 rows, slower from 1024).  Both kernels sum the
// row statistics in the same order, so the switch changes no bits.
constexpr int64_t kTableLdsMinRows = 513;

// FULL as for k_adaln_fp8_rows.
template <int VPT, int WAVES, int R = kTableRows, bool MX = false, bool FULL = false>
__global__ __launch_bounds__(R * WAVES * 64) void k_adaln_fp8_table_lds(Fp8Args a)
{
    extern __shared__ float4 tab[];   // [0, dim/4): scale row, [dim/4, dim/2): shift row
    __shared__ float red[2][R * WAVES];
    constexpr int T = WAVES * 64;      // threads per row
    constexpr int NT = R * T;          // threads per workgroup
    const int tid = threadIdx.x;
    const int rr = tid / T, t = tid % T;
    const int dim = a.dim;
    const int nvec = dim >> 3;
    const int n4 = dim >> 2;
    const float inv = MX ? 0.f : 1.0f / *a.act_scale;
    const int64_t row = grid_row() * R + rr;
    const bool valid = row < a.rows;
    ALNP_TL_VARS;
    ALNP_TL_MARK(0);

    // The table rows: up to 8 float4 per thread in flight, the rest (only for
    // dims above 4 * 2 * NT ... 8192) loaded while they are written to LDS.
    // Where they are requested depends on the output format (XFIRST below).
    const float4* tsrc = reinterpret_cast<const float4*>(a.table + (int64_t)a.scale_idx * dim);
    const float4* thsrc = reinterpret_cast<const float4*>(a.table + (int64_t)a.shift_idx * dim);
    constexpr int kFirst = 8;
    float4 tv[kFirst];
    // XFIRST (FP8): the row's x is requested first and the table rows only
    // once x has landed; they go to LDS before the second reduction, whose
    // barrier publishes them.  Requested ahead of x, the table loads of the
    // first workgroups on a CU (24 KiB each, L2 hits) hold up the issue of
    // the later workgroups' x by microseconds (per-wave timestamps: the
    // fourth and fifth workgroups of a CU got x 2-4 us after the first
    // three).  2520 x 3072 cold: 10.97 -> 10.81 us, bit-identical.  MXFP8
    // keeps the table ahead of x, which measured better there (11.17
    // against 11.37 us), with the table in LDS before the first reduction.
    constexpr bool XFIRST = !MX;
    if (!XFIRST) {
#pragma unroll
        for (int k = 0; k < kFirst; ++k) {
            const int idx = tid + k * NT;  // over the 2 * n4 table vectors
            tv[k] = idx < n4 ? tsrc[idx] : idx < 2 * n4 ? thsrc[idx - n4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }

    const int64_t lrow = valid ? row : 0;
    const uint16_t* xr = a.x + lrow * dim;
    const uint16_t* scr = a.temb + (lrow * a.chunks + a.scale_idx) * dim;
    const uint16_t* shr = a.temb + (lrow * a.chunks + a.shift_idx) * dim;
    // A workgroup's second row past the end (odd row counts) computes on row 0
    // and stores nothing.
    uint4 xv[VPT], scv[VPT], shv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        xv[v] = ld_row<true>(xr, v * T + t, nvec, !FULL && v == VPT - 1);
    ALNP_TL_MARK(1);
    // The temb chunks are requested after the first reduction (FP8) or the
    // second (MXFP8), as in k_adaln_fp8_rows; those points measured best
    // for this kernel (2520 x 3072 cold: FP8 11.33 -> 10.95 us, MXFP8 11.42
    // -> 11.14 us).
    constexpr int kLoad = MX ? kAfterRstd : kAfterMean;
    auto load_streamed = [&](int when) {
        if (when != kLoad)
            return;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            scv[v] = ld_row<true>(scr, v * T + t, nvec, !FULL && v == VPT - 1);
            shv[v] = ld_row<true>(shr, v * T + t, nvec, !FULL && v == VPT - 1);
        }
    };
    load_streamed(kWithX);

    // Row statistics over the row's WAVES waves (the barriers also publish
    // the LDS table).
    const bool tail_ok = FULL || (VPT - 1) * T + t < nvec;
    auto reduce = [&](float v, int k) { return subgroup_sum(v, red[k], rr * WAVES, WAVES); };
    float d[VPT][8];
    float mean, rstd;
    if (XFIRST) {
        const float s = thread_sum<VPT>(xv);
        ALNP_TL_MARK_AFTER(2, s);
        // The table loads after x has landed (the sum needs it): without
        // the pin the scheduler hoists them back above the sum.
        asm volatile("" ::"v"(s));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kFirst; ++k) {
            const int idx = tid + k * NT;  // over the 2 * n4 table vectors
            tv[k] = idx < n4 ? tsrc[idx] : idx < 2 * n4 ? thsrc[idx - n4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        mean = reduce(s, 0) * a.inv_dim;
        load_streamed(kAfterMean);
        const float q = thread_sumsq<VPT>(xv, tail_ok, mean, d);
#pragma unroll
        for (int k = 0; k < kFirst; ++k) {
            const int idx = tid + k * NT;
            if (idx < 2 * n4)
                tab[idx] = tv[k];
        }
        for (int idx = tid + kFirst * NT; idx < 2 * n4; idx += NT)
            tab[idx] = idx < n4 ? tsrc[idx] : thsrc[idx - n4];
        rstd = rsqrt_refined(reduce(q, 1) * a.inv_dim + a.eps);
    } else {
#pragma unroll
        for (int k = 0; k < kFirst; ++k) {
            const int idx = tid + k * NT;
            if (idx < 2 * n4)
                tab[idx] = tv[k];
        }
        for (int idx = tid + kFirst * NT; idx < 2 * n4; idx += NT)
            tab[idx] = idx < n4 ? tsrc[idx] : thsrc[idx - n4];
        const float s = thread_sum<VPT>(xv);
        ALNP_TL_MARK_AFTER(2, s);
        mean = reduce(s, 0) * a.inv_dim;
        load_streamed(kAfterMean);
        rstd = row_rstd<VPT>(xv, tail_ok, mean, a.inv_dim, a.eps, reduce, d);
    }
    ALNP_TL_MARK_AFTER(3, rstd);
    load_streamed(kAfterRstd);
    if (!valid)
        return;

#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * T + t;
        if (v == VPT - 1 && !tail_ok)
            continue;
        float sc[8], sh[8];
        unpack8(scv[v], sc);
        unpack8(shv[v], sh);
        const float4 s0 = tab[2 * i], s1 = tab[2 * i + 1];
        const float4 h0 = tab[n4 + 2 * i], h1 = tab[n4 + 2 * i + 1];
        const float ts[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float th[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        float q8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float scale = sc[e] + ts[e];
            const float shift = sh[e] + th[e];
            const float xhat = d[v][e] * rstd;
            const float y = (xhat * (1.0f + scale)) + shift;
            q8[e] = MX ? y : y * inv;
        }
        if (!MX)
            sat448x8(q8);
        if (MX) {
            // MXFP8: as in k_adaln_fp8_rows (a quad of lanes holds one block).
            const int E = mx_scale_exp(quad_max(absmax8(q8)), 8);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                q8[e] = sat448(__builtin_amdgcn_ldexpf(q8[e], -E));
            a.mx_scales[row * (dim >> 5) + (i >> 2)] = (uint8_t)(E + 127);
        }
        st_stream(a.out + row * dim + (int64_t)i * 8,
                  make_uint2(pack_e4m3x4(q8[0], q8[1], q8[2], q8[3]),
                             pack_e4m3x4(q8[4], q8[5], q8[6], q8[7])));
    }
    if (t == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
    ALNP_TL_MARK(4);
    ALNP_TL_RECORD(row, WAVES);
}

__global__ __launch_bounds__(256) void k_adaln_fp8_block(Fp8Args a, int form)
{
    __shared__ float lds4[4];
    const int dim = a.dim;
    const float inv = 1.0f / *a.act_scale;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const uint16_t* xr = a.x + row * dim;
    float mean, rstd;
    block_row_stats(xr, dim, a.inv_dim, a.eps, lds4, mean, rstd);
    for (int j = threadIdx.x; j < dim; j += 256) {
        float sc = 0.f, sh = 0.f;
        if (form == kBcast) {
            sc = ldbf(a.scale, j);
            sh = ldbf(a.shift, j);
        } else if (form == kPtok) {
            sc = ldbf(a.scale, row * dim + j);
            sh = ldbf(a.shift, row * dim + j);
        } else if (form == kTable) {
            sc = ldbf(a.temb, (row * a.chunks + a.scale_idx) * dim + j) +
                 a.table[(int64_t)a.scale_idx * dim + j];
            sh = ldbf(a.temb, (row * a.chunks + a.shift_idx) * dim + j) +
                 a.table[(int64_t)a.shift_idx * dim + j];
        } else if (form == kModFp8) {
            sc = __builtin_amdgcn_cvt_f32_fp8((int)a.scale_fp8[j], 0) * *a.scale_deq;
            sh = __builtin_amdgcn_cvt_f32_fp8((int)a.shift_fp8[j], 0) * *a.shift_deq;
        } else if (form == kAwq) {
            sc = ldbf(a.scale, j);
            sh = ldbf(a.shift, j);
        }
        const float xhat = (ldbf(xr, j) - mean) * rstd;
        float y = (xhat * (1.0f + sc)) + sh;
        if (form == kAwq)
            y = y * ldbf(a.inv_s, j);
        a.out[row * dim + j] = (uint8_t)(pack_e4m3x4(sat448(y * inv), 0.f, 0.f, 0.f) & 0xFFu);
    }
    if (threadIdx.x == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
    }
}

// MX fallbacks: one workgroup per row, one thread per 32-element block.
__global__ __launch_bounds__(256) void k_mxfp8_block(Fp8Args a, int form)
{
    __shared__ float lds4[4];
    const int dim = a.dim;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const uint16_t* xr = a.x + row * dim;
    float mean, rstd;
    block_row_stats(xr, dim, a.inv_dim, a.eps, lds4, mean, rstd);
    for (int k = threadIdx.x; k < dim / 32; k += 256) {
        float y[32];
        float amax = 0.f;
        for (int e = 0; e < 32; ++e) {
            const int j = 32 * k + e;
            float sc = 0.f, sh = 0.f;
            if (form == kBcast) {
                sc = ldbf(a.scale, j);
                sh = ldbf(a.shift, j);
            } else if (form == kPtok) {
                sc = ldbf(a.scale, row * dim + j);
                sh = ldbf(a.shift, row * dim + j);
            } else if (form == kTable) {
                sc = ldbf(a.temb, (row * a.chunks + a.scale_idx) * dim + j) +
                     a.table[(int64_t)a.scale_idx * dim + j];
                sh = ldbf(a.temb, (row * a.chunks + a.shift_idx) * dim + j) +
                     a.table[(int64_t)a.shift_idx * dim + j];
            } else if (form == kModFp8) {
                sc = __builtin_amdgcn_cvt_f32_fp8((int)a.scale_fp8[j], 0) * *a.scale_deq;
                sh = __builtin_amdgcn_cvt_f32_fp8((int)a.shift_fp8[j], 0) * *a.shift_deq;
            } else if (form == kAwq) {
                sc = ldbf(a.scale, j);
                sh = ldbf(a.shift, j);
            }
            const float xhat = (ldbf(xr, j) - mean) * rstd;
            y[e] = (xhat * (1.0f + sc)) + sh;
            if (form == kAwq)
                y[e] = y[e] * ldbf(a.inv_s, j);
            amax = fmaxf(amax, fabsf(y[e]));
        }
        const int E = mx_scale_exp(amax, 8);
        for (int e = 0; e < 32; ++e)
            a.out[row * dim + 32 * k + e] =
                (uint8_t)(pack_e4m3x4(sat448(__builtin_amdgcn_ldexpf(y[e], -E)), 0.f, 0.f, 0.f) & 0xFFu);
        a.mx_scales[row * (dim / 32) + k] = (uint8_t)(E + 127);
    }
    if (threadIdx.x == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
    }
}

// ---- standalone quantizer ---------------------------------------------------

__global__ __launch_bounds__(256) void k_quant_fp8(const float* v, const float* act, int64_t n,
                                                   uint8_t* out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const float inv = 1.0f / *act;
    out[i] = (uint8_t)(pack_e4m3x4(sat448(v[i] * inv), 0.f, 0.f, 0.f) & 0xFFu);
}

// ---- launchers ----------------------------------------------------------------

RowShape row_shape(int dim)
{
    // Waves per row (1, 2, 4 or 8) and 16-byte vectors per thread (1..8) for
    // a row of dim/8 vectors: the least padding, with 2-4 vectors per thread
    // preferred (fewer waves and barriers than 1, shorter per-wave tails than
    // 5-8), then 3.
    const int nvec = dim / 8;
    RowShape best{0, 0};
    double best_score = 1e30;
    for (int vpt = 1; vpt <= 8; ++vpt) {
        int waves = 1;
        while (waves * 64 * vpt < nvec && waves < 8)
            waves *= 2;
        if (waves * 64 * vpt < nvec || (vpt - 1) * waves * 64 > nvec)
            continue;  // too short, or more than the last slot past the end
        const double waste = double(waves * 64 * vpt - nvec) / nvec;
        const double score = waste + (vpt == 1 ? 0.1 : vpt > 4 ? 0.02 * (vpt - 4) : 0.0) +
                             (vpt == 3 ? -1e-3 : 0.0);
        if (score < best_score) {
            best_score = score;
            best = RowShape{waves * 64, vpt};
        }
    }
    return best;
}

// From this many rows the broadcast, modfp8 and AWQ forms form their shared
// operands ahead of the row (k_adaln_fp8_rows, PRE).  Smaller calls are
// latency-bound: there the operand loads ahead of x delay the row more than
// the shorter output pass saves (broadcast 16 x 2048: 2.87 -> 3.01 us).
// Both orders compute the same bits.
constexpr int64_t kPreMinRows = 512;

template <int FORM, bool MX, bool PRE, bool PAIRS = false>
static hipError_t launch_fp8_rows_as(const Fp8Args& a, RowShape rs, hipStream_t s)
{
    const dim3 grid = row_grid(a.rows);
    if ((a.dim >> 3) == rs.vpt * rs.threads) {
#define ALNP_LAUNCH(V, W)                                                                           \
    hipLaunchKernelGGL((k_adaln_fp8_rows<V, W, FORM, MX, true, PRE && V <= 3, PAIRS && PRE && V <= 3>), \
                       grid, dim3(W * 64), 0, s, a)
        ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
        return hipGetLastError();
    }
#define ALNP_LAUNCH(V, W) \
    hipLaunchKernelGGL((k_adaln_fp8_rows<V, W, FORM, MX, false, PRE && V <= 3>), grid, dim3(W * 64), 0, s, a)
    ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
    return hipGetLastError();
}

template <int FORM, bool MX = false>
static hipError_t launch_fp8_rows(const Fp8Args& a, RowShape rs, hipStream_t s)
{
    constexpr bool kShared = FORM == kBcast || FORM == kModFp8 || FORM == kAwq;
    if (kShared && a.rows >= kPreMinRows) {
        constexpr bool kPairs = FORM == kModFp8 && !MX;
        if (kPairs && ((reinterpret_cast<uintptr_t>(a.scale_fp8) |
                        reinterpret_cast<uintptr_t>(a.shift_fp8)) & 15) == 0)
            return launch_fp8_rows_as<FORM, MX, kShared, kPairs>(a, rs, s);
        return launch_fp8_rows_as<FORM, MX, kShared>(a, rs, s);
    }
    return launch_fp8_rows_as<FORM, MX, false>(a, rs, s);
}

// The LDS table kernel runs rows of at most 4 waves (its caller checks), so
// the 8-wave shapes are not instantiated.
template <int V, int W>
static void launch_table_lds_shape(const Fp8Args& a, dim3 grid, size_t lds, hipStream_t s)
{
    if constexpr (W <= 4) {
        if ((a.dim >> 3) == V * W * 64)
            hipLaunchKernelGGL((k_adaln_fp8_table_lds<V, W, kTableRows, false, true>), grid,
                               dim3(kTableRows * W * 64), lds, s, a);
        else
            hipLaunchKernelGGL((k_adaln_fp8_table_lds<V, W>), grid, dim3(kTableRows * W * 64), lds, s, a);
    }
}

static hipError_t launch_fp8_table_lds(const Fp8Args& a, RowShape rs, hipStream_t s)
{
    const dim3 grid = row_grid((a.rows + kTableRows - 1) / kTableRows);
    const size_t lds = 2 * (size_t)a.dim * sizeof(float);
#define ALNP_LAUNCH(V, W) launch_table_lds_shape<V, W>(a, grid, lds, s)
    ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
    return hipGetLastError();
}

hipError_t launch_adaln_fp8(const Fp8Args& args, int form, bool fast, hipStream_t s)
{
    Fp8Args a = args;
    a.inv_dim = 1.0f / (float)a.dim;
    const RowShape rs = fast ? row_shape(a.dim) : RowShape{0, 0};
    if (rs.vpt > 0 && form == kTable && a.dim <= kTableMaxDim && rs.threads <= 256 &&
        a.rows >= kTableLdsMinRows)
        return launch_fp8_table_lds(a, rs, s);
    if (rs.vpt > 0) {
        switch (form) {
        case kNone: return launch_fp8_rows<kNone>(a, rs, s);
        case kBcast: return launch_fp8_rows<kBcast>(a, rs, s);
        case kPtok: return launch_fp8_rows<kPtok>(a, rs, s);
        case kTable: return launch_fp8_rows<kTable>(a, rs, s);
        case kModFp8: return launch_fp8_rows<kModFp8>(a, rs, s);
        case kAwq: return launch_fp8_rows<kAwq>(a, rs, s);
        default: return hipErrorInvalidValue;
        }
    }
    const dim3 grid((unsigned)std::min<int64_t>(a.rows, kMaxGrid));
    hipLaunchKernelGGL(k_adaln_fp8_block, grid, dim3(256), 0, s, a, form);
    return hipGetLastError();
}

template <int FORM>
static hipError_t launch_mxfp8_rows(const Fp8Args& a, RowShape rs, hipStream_t s)
{
    return launch_fp8_rows<FORM, true>(a, rs, s);
}

template <int V, int W>
static void launch_table_lds_mx_shape(const Fp8Args& a, dim3 grid, size_t lds, hipStream_t s)
{
    if constexpr (W <= 4) {
        if ((a.dim >> 3) == V * W * 64)
            hipLaunchKernelGGL((k_adaln_fp8_table_lds<V, W, kTableRows, true, true>), grid,
                               dim3(kTableRows * W * 64), lds, s, a);
        else
            hipLaunchKernelGGL((k_adaln_fp8_table_lds<V, W, kTableRows, true>), grid,
                               dim3(kTableRows * W * 64), lds, s, a);
    }
}

hipError_t launch_mxfp8(const Fp8Args& args, int form, bool fast, hipStream_t s)
{
    Fp8Args a = args;
    a.inv_dim = 1.0f / (float)a.dim;
    const RowShape rs = fast ? row_shape(a.dim) : RowShape{0, 0};
    if (rs.vpt > 0 && form == kTable && a.dim <= kTableMaxDim && rs.threads <= 256 &&
        a.rows >= kTableLdsMinRows) {
        const dim3 grid = row_grid((a.rows + kTableRows - 1) / kTableRows);
        const size_t lds = 2 * (size_t)a.dim * sizeof(float);
#define ALNP_LAUNCH(V, W) launch_table_lds_mx_shape<V, W>(a, grid, lds, s)
        ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
        return hipGetLastError();
    }
    if (rs.vpt > 0) {
        switch (form) {
        case kNone: return launch_mxfp8_rows<kNone>(a, rs, s);
        case kBcast: return launch_mxfp8_rows<kBcast>(a, rs, s);
        case kPtok: return launch_mxfp8_rows<kPtok>(a, rs, s);
        case kTable: return launch_mxfp8_rows<kTable>(a, rs, s);
        case kModFp8: return launch_mxfp8_rows<kModFp8>(a, rs, s);
        case kAwq: return launch_mxfp8_rows<kAwq>(a, rs, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (form < kNone || form > kAwq)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)std::min<int64_t>(a.rows, kMaxGrid));
    hipLaunchKernelGGL(k_mxfp8_block, grid, dim3(256), 0, s, a, form);
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const float* v, const float* act, int64_t n, uint8_t* out,
                            hipStream_t s)
{
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_quant_fp8, dim3((unsigned)blocks), dim3(256), 0, s, v, act, n, out);
    return hipGetLastError();
}

}  // namespace alnp

#ifdef ALNP_TIMELINE
// Measurement-only build: the buffer the FP8 row and table kernels write
// their per-wave records to (timeline.hpp).  Not part of the product ABI.
__device__ unsigned long long* alnp::timeline_buf;

extern "C" int alnp_timeline_set(void* buf)
{
    return hipMemcpyToSymbol(HIP_SYMBOL(alnp::timeline_buf), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#endif

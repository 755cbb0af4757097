// W4A4 GEMM on INT8 MFMA with W4 nibble unpack into LDS and a fused
// scale / bias / cast epilogue (gfx950).
//
// What is computed (web page "[Feat][Ascend] Consolidate INT8, RotateQuant,
// RoPE and ConvRot W4A4 backends", section "W4A4 correctness and performance
// scope"; per-64-group weight scales and the low-rank term from the source
// page comfy_kitchen/tensor/svdquant_w4a4.py, module docstring):
//   acc[m,n] = sum_k c[m,k] * w[n,k]                 exact integer sum
//   out[m,n] = O( ((f32(acc) * s_a[m]) * s_w[n]) [+ l[m,n]] [+ bias[n]] )
// or, with per-64-group weight scales,
//   out[m,n] = O( ((sum_G f32(acc_G) * s_w[G,n]) * s_a[m]) [+ l] [+ bias] )
// with l[m,n] = sum_r L[m,r] * up[n,r]; every listed multiply and add is a
// separately rounded fp32 operation.
//
// Design for CDNA4 (three kernels; launch_gemm picks one per call):
//   * w4a4_gemm_ring3_kernel, for prefill-sized layers: persistent, one
//     workgroup per CU walking 256 x 256 output tiles; eight waves, two per
//     SIMD, each a 128 x 64 block of 8 x 4 v_mfma_i32_16x16x64_i8 tiles with
//     its 128 INT32 accumulators in VGPRs.  Codes and packed weights stream
//     global -> LDS through buffer_load ... lds into a three-stage ring, so two
//     K-steps are in flight while one is multiplied; the weights are unpacked
//     in registers right before the MFMAs.
//   * w4a4_gemm_skinny_kernel, for decode-sized M (<= 64): one 1024-thread
//     workgroup per 16 output columns; its sixteen waves split K and their
//     INT32 tiles are summed exactly in LDS.
//   * w4a4_gemm_kernel, for everything else (per-64-group weight scales, the
//     low-rank term with group scales, INT32 export, K-chunked runs, M <= 128):
//     128 x 128 output tile, 4 waves in 2 x 2, each a 64 x 64 block of 4 x 4
//     MFMA tiles; K advances 64 per step with double-buffered LDS and the next
//     step's global loads in flight during the MFMAs.  With group scales each
//     step's INT32 tile is converted and accumulated in fp32 in the order
//     above, with the group's scales staged through LDS alongside the operands.
//   * Packed weights are read as bytes (N, K/2) and unpacked as 16*w: the low
//     nibble shifted into the high half of a byte and the high nibble masked
//     in place are both already sign-correct int8 values, so unpacking is
//     shift/and/perm with no sign extension.  The integer result is divided
//     by 16 (an exact arithmetic shift) before the epilogue.
//   * Workgroups are dealt round-robin over the 8 XCDs; tiles are renumbered
//     so that each XCD works on a contiguous, M-grouped range and its L2 sees
//     shared code rows and weight columns.
//   * When K is too large for INT32 (16 * 7 * 8 * K > 2^31 - 1) or a chunk
//     size is forced, each workgroup accumulates one K-chunk and adds it into
//     an int64 workspace with 64-bit atomics (exact and order-independent);
//     a second kernel applies the epilogue.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace w4a4 {

constexpr int BM = 128, BN = 128, BK = 64, LDR = 80;
__device__ __forceinline__ void unpack16(uint32_t p, uint32_t& lo4, uint32_t& hi4)
{
    // p holds 8 nibbles for k0..k7 (even k in the low nibble of each byte).
    const uint32_t L = (p << 4) & 0xf0f0f0f0u;  // 16*w(k0), 16*w(k2), 16*w(k4), 16*w(k6)
    const uint32_t H = p & 0xf0f0f0f0u;         // 16*w(k1), 16*w(k3), ...
    lo4 = __builtin_amdgcn_perm(H, L, 0x05010400u);  // k0 k1 k2 k3
    hi4 = __builtin_amdgcn_perm(H, L, 0x07030602u);  // k4 k5 k6 k7
}

__device__ __forceinline__ float epilogue_tail(float t, const GemmArgs& a, int64_t row, int64_t col)
{
    if (a.lora) {
        const float* lr = a.lora + row * a.rank;
        float l = 0.0f;
        for (int r = 0; r < a.rank; ++r)
            l = fmaf(lr[r], load_any_f32(a.up_dtype, a.up, col * a.rank + r), l);
        t = add_rn(t, l);
    }
    if (a.bias) t = add_rn(t, load_any_f32(a.bias_dtype, a.bias, col));
    return t;
}

// Buffer resource over `bytes` bytes at `base`: loads past the end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}

// GSW: -1 for one weight scale per column, else the dtype of the per-64-group
// weight scales (F32, F16 or BF16)
template <int GSW, bool SPLIT, bool ALIGNED>
__global__ __launch_bounds__(256) void w4a4_gemm_kernel(GemmArgs a, int64_t kc)
{
    constexpr bool GROUP = GSW >= 0;
    __shared__ __align__(16) int8_t As[2][BM * LDR];
    __shared__ __align__(16) int8_t Bs[2][BN * LDR];
    __shared__ __align__(16) float Ss[GSW >= 0 ? 2 : 1][GSW >= 0 ? 256 : 4];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    // Workgroups are dealt round-robin over the 8 XCDs; give each XCD a
    // contiguous range of tiles, M-grouped, so its L2 sees shared code rows and
    // weight columns.
    const int tiles_n = (int)gridDim.x, tiles_m = (int)gridDim.y;
    const int ntiles = tiles_m * tiles_n;
    const int bid = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    const int q8 = ntiles >> 3, r8 = ntiles & 7;
    const int xcd = bid & 7, loc = bid >> 3;
    const int tile = xcd * q8 + min(xcd, r8) + loc;
    constexpr int GROUP_M = 16;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile - (tile / per_group) * per_group;
    const int64_t m0 = (int64_t)(first_m + in_g % gsize) * BM;
    const int64_t n0 = (int64_t)(in_g / gsize) * BN;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int64_t kbeg = (int64_t)blockIdx.z * kc;
    const int64_t kend = min(K, kbeg + kc);
    const int nsteps = (int)((kend - kbeg + BK - 1) / BK);

    // global -> register staging
    uint4 ra[2];
    uint4 rw;
    // ALIGNED without K-chunks (K % 64 == 0): buffer loads over the tile's
    // code rows and weight columns, fixed lane offsets plus the step's k as the
    // scalar offset; rows past M and columns past N read zeros (a load past
    // the last step reads the next row, and only fills the idle buffer)
    constexpr bool BUF = ALIGNED && !SPLIT;
    const __amdgpu_buffer_rsrc_t rca =
        make_rsrc(a.codes + (m0 < M ? m0 : 0) * K, (uint64_t)(m0 < M ? min(M - m0, (int64_t)BM) : 0) * K);
    const __amdgpu_buffer_rsrc_t rcw = make_rsrc(
        a.wp + (n0 < N ? n0 : 0) * (K >> 1), (uint64_t)(n0 < N ? min(N - n0, (int64_t)BN) : 0) * (K >> 1));
    auto gload = [&](int64_t k) {
        if constexpr (BUF) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = tid + 256 * i;
                ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    rca, (int)((c >> 2) * K + (c & 3) * 16), (int)k, 0));
            }
            rw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rcw, (int)((tid >> 1) * (K >> 1) + (tid & 1) * 16), (int)(k >> 1), 0));
            return;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, c16 = c & 3;
            const int64_t gm = m0 + row, gk = k + c16 * 16;
            if constexpr (ALIGNED) {
                if (gm < M && gk < kend) ra[i] = *(const uint4*)(a.codes + gm * K + gk);
                else ra[i] = make_uint4(0, 0, 0, 0);
            } else {
                uint32_t wv[4] = {0, 0, 0, 0};
                if (gm < M)
                    for (int e = 0; e < 16; ++e)
                        if (gk + e < kend)
                            wv[e >> 2] |= (uint32_t)(uint8_t)a.codes[gm * K + gk + e] << (8 * (e & 3));
                ra[i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
        }
        const int n = tid >> 1, half = tid & 1;
        const int64_t gn = n0 + n;
        const int64_t kp = (k >> 1) + half * 16;  // packed byte index
        if constexpr (ALIGNED) {
            if (gn < N && 2 * kp < kend) rw = *(const uint4*)(a.wp + gn * (K >> 1) + kp);
            else rw = make_uint4(0, 0, 0, 0);
        } else {
            uint32_t wv[4] = {0, 0, 0, 0};
            if (gn < N)
                for (int e = 0; e < 16; ++e)
                    if (2 * (kp + e) < kend)
                        wv[e >> 2] |= (uint32_t)a.wp[gn * (K >> 1) + kp + e] << (8 * (e & 3));
            rw = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, c16 = c & 3;
            *(uint4*)(&As[buf][row * LDR + c16 * 16]) = ra[i];
        }
        const int n = tid >> 1, half = tid & 1;
        uint4 u0, u1;
        unpack16(rw.x, u0.x, u0.y);
        unpack16(rw.y, u0.z, u0.w);
        unpack16(rw.z, u1.x, u1.y);
        unpack16(rw.w, u1.z, u1.w);
        *(uint4*)(&Bs[buf][n * LDR + half * 32]) = u0;
        *(uint4*)(&Bs[buf][n * LDR + half * 32 + 16]) = u1;
    };

    v4i acc[4][4];
    v4f facc[GROUP ? 4 : 1][GROUP ? 4 : 1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};
    if constexpr (GROUP) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) facc[mt][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
    }

    // The K loop. With group scales the MFMA sums carry the weights' factor
    // 16 (high-nibble unpack); FAST multiplies float(16 s) by scale / 16,
    // which is the same real number as s * scale and so rounds to the same
    // float, whenever scale / 16 is exact (every scale but subnormal or NaN
    // ones). It returns false if some scale was not; the workgroup then runs
    // the loop again with the shift back to s.
    auto kloop = [&](auto fast_c) -> bool {
        constexpr bool FAST = decltype(fast_c)::value;
        bool exact = true;
        // Group scales ride the operand pipeline: thread t loads the scale of
        // column c(t) = (t / 64 % 2) * 64 + (t % 4) * 16 + (t / 4) % 16 with its
        // step's operands and stores it to LDS at slot t (FAST: divided by 16
        // and checked), so that a lane's four columns are one 16-byte read.
        // Threads 128..255 repeat threads 0..127 (no branch: a branch here
        // lets the compiler sink the MFMA conversions past the operand wait).
        // Columns past N read column N - 1 and steps past the end the last
        // group: those values are never used.
        uint32_t rsw = 0;
        const int scl = ((tid >> 6) & 1) * 64 + (tid & 3) * 16 + ((tid >> 2) & 15);
        const uint32_t sc = (uint32_t)min(n0 + scl, N - 1);
        auto sgload = [&](int step) {
            if constexpr (GROUP) {
                const int64_t gidx = min((kbeg + (int64_t)step * BK) / 64, (K + 63) / 64 - 1);
                if constexpr (GSW == F32) rsw = ((const uint32_t*)a.sw + gidx * N)[sc];
                else rsw = ((const uint16_t*)a.sw + gidx * N)[sc];
            }
        };
        auto ssstore = [&](int buf) {
            if constexpr (GROUP) {
                const float v = GSW == F32 ? __uint_as_float(rsw) : h_to_f32<GSW>((uint16_t)rsw);
                float w = v;
                if constexpr (FAST) {
                    w = v * 0.0625f;
                    exact = exact && w * 16.0f == v;
                }
                Ss[buf][tid] = w;
            }
        };
        if (nsteps > 0) {
            sgload(0);
            gload(kbeg);
            sstore(0);
            ssstore(0);
        }
        __syncthreads();
        for (int s = 0; s < nsteps; ++s) {
            const int buf = s & 1;
            // (past the last step the loads are masked off and the stores
            // fill the idle buffer with zeros: no branch in the loop)
            sgload(s + 1);
            gload(kbeg + (int64_t)(s + 1) * BK);
            v4i af[4], bf[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                af[mt] = *(const v4i*)(&As[buf][(wm * 64 + mt * 16 + j) * LDR + q * 16]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                bf[nt] = *(const v4i*)(&Bs[buf][(wn * 64 + nt * 16 + j) * LDR + q * 16]);
            if constexpr (GROUP) {
                const v4f swv = *(const v4f*)(&Ss[buf][(wn * 16 + j) * 4]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        v4i t = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], (v4i){0, 0, 0, 0},
                                                                      0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            facc[mt][nt][r] = add_rn(facc[mt][nt][r],
                                                     mul_rn((float)(FAST ? t[r] : t[r] >> 4), swv[nt]));
                    }
                if constexpr (FAST) {
                    // one MFMA, then twelve VALU instructions (converting an
                    // earlier result), sixteen times
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
                    }
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], acc[mt][nt],
                                                                            0, 0, 0);
            }
            // (keep the stores after the MFMAs and conversions: they wait for
            // this step's loads)
            __builtin_amdgcn_sched_barrier(0);
            sstore(buf ^ 1);
            ssstore(buf ^ 1);
            __syncthreads();
        }
        return exact;
    };
    if constexpr (GROUP) {
        if (__syncthreads_or(!kloop(std::true_type{}))) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) facc[mt][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
            kloop(std::false_type{});
        }
    } else {
        kloop(std::false_type{});
    }

    // ---- low-rank term (rank <= 32): the tile's rows of L and columns of
    // proj_up go to LDS as fp32 (the staging buffers are free after the loop;
    // ranks padded with zeros to a multiple of 4), and each lane sums
    // l[m,n] = sum_r L[m,r] * up[n,r] for its outputs, one row block at a
    // time, in increasing r with fmaf, four terms per read: the same
    // operations as epilogue_tail
    constexpr int LDL = 36;  // fp32 row stride: 16-byte reads of 16 columns hit distinct banks
    static_assert(BM * LDL * 4 <= 2 * BM * LDR && BN * LDL * 4 <= 2 * BN * LDR, "low-rank staging");
    const bool lds_lora = !SPLIT && a.lora != nullptr && a.rank >= 1 && a.rank <= 32;
    const float* Ls = (const float*)&As[0][0];
    const float* Us = (const float*)&Bs[0][0];
    const int RP = (a.rank + 3) & ~3;
    if (lds_lora) {
        float* Lw = (float*)&As[0][0];
        float* Uw = (float*)&Bs[0][0];
        const int R = a.rank;
        for (int i = tid; i < BM * RP; i += 256) {
            const int rr = i / RP, c = i - rr * RP;
            const int64_t gm = m0 + rr;
            Lw[rr * LDL + c] = (gm < M && c < R) ? a.lora[gm * R + c] : 0.0f;
        }
        for (int i = tid; i < BN * RP; i += 256) {
            const int cc = i / RP, c = i - cc * RP;
            const int64_t gn = n0 + cc;
            Uw[cc * LDL + c] = (gn < N && c < R) ? load_any_f32(a.up_dtype, a.up, gn * R + c) : 0.0f;
        }
        __syncthreads();
    }

    // ---- epilogue: lane (j, q) holds rows 4q..4q+3, column j of each tile.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        float lsum[4][4];
        if (lds_lora) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) lsum[nt][r] = 0.0f;
            for (int c4 = 0; c4 < RP; c4 += 4) {
                v4f lr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    lr[r] = *(const v4f*)(Ls + (wm * 64 + mt * 16 + 4 * q + r) * LDL + c4);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const v4f u = *(const v4f*)(Us + (wn * 64 + nt * 16 + j) * LDL + c4);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int e = 0; e < 4; ++e) lsum[nt][r] = fmaf(lr[r][e], u[e], lsum[nt][r]);
                }
            }
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + mt * 16 + 4 * q + r;
                const int64_t col = n0 + wn * 64 + nt * 16 + j;
                if (row >= M || col >= N) continue;
                if constexpr (SPLIT) {
                    atomicAdd((unsigned long long*)(a.acc64 + row * N + col),
                              (unsigned long long)(int64_t)(acc[mt][nt][r] >> 4));
                } else {
                    float t;
                    if constexpr (GROUP) {
                        t = mul_rn(facc[mt][nt][r], a.sa[row]);
                    } else {
                        const int32_t iv = acc[mt][nt][r] >> 4;
                        if (a.acc_out) a.acc_out[row * N + col] = iv;
                        t = (float)iv;
                        t = mul_rn(t, a.sa[row]);
                        t = mul_rn(t, load_any_f32(a.sw_dtype, a.sw, col));
                    }
                    if (lds_lora) {
                        t = add_rn(t, lsum[nt][r]);
                        if (a.bias) t = add_rn(t, load_any_f32(a.bias_dtype, a.bias, col));
                    } else {
                        t = epilogue_tail(t, a, row, col);
                    }
                    store_any(a.out_dtype, a.out, row * N + col, t);
                }
            }
    }
}



constexpr int BBM = 256, BBN = 256;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));


// -------------------------------------------------------------------------
// Three-stage persistent kernel (per-channel scales, M > 128, K % 128 == 0):
// one 512-thread workgroup per CU walks its 256 x 256 output tiles; eight
// waves in 2 (M) x 4 (N), two per SIMD, each a 128 x 64 block of 8 x 4
// v_mfma_i32_16x16x64_i8 tiles with its 128 INT32 accumulators in VGPRs; K
// advances 128 per step.
//   * Codes (32 KB per step) and packed weights (16 KB per step) go global ->
//     LDS with buffer_load ... lds (no VGPR staging) into a ring of three
//     48 KB slots.  The ring runs across tiles: the last two steps of a tile
//     fetch the first two stages of the workgroup's next tile, and the
//     epilogue of a tile works in the slot its last step freed, so output
//     stores overlap the next tile's loads.
//   * Codes keep 128-byte rows; eight consecutive fetch lanes read one row's
//     K-slice, so each load instruction covers eight whole 128-byte segments.
//     16-byte chunk c of row r sits at c ^ r3_swz(r).  On gfx950 a
//     ds_read_b128 serves the 64 lanes in four cycles, two per pair of 16-lane
//     groups, split by lane index j (group g lanes with j in {0-3, 12-15}
//     together with group g+1 lanes with j in {4-11}), over 64 four-byte
//     banks; with this swizzle the fragment reads of both k-substeps hit 16
//     distinct 16-byte bank groups in every cycle.
//   * Packed weights keep their 64-byte rows (one per output column), 16-byte
//     chunk c of column n stored at c ^ ((n >> 1) & 3), which spreads a
//     fragment read over all banks.
//   * Every byte offset, row and k included, travels in the per-lane voffset,
//     so the buffer range check covers it: rows past M or N and k past K read
//     as zero, and a missing next tile is a zero-sized buffer.
//   * Every step waits only for its own stage (vmcnt leaves the next stage's
//     loads in flight), meets the other waves at a bare s_barrier
//     (__syncthreads would also wait for the loads still in flight) and then
//     puts stage s+2 in flight before computing stage s.
//   * Two waves per SIMD keep the matrix core busy while the other waits on
//     LDS or the barrier; with at most 256 registers per lane the compiler
//     keeps the accumulators in VGPRs, where every MFMA updates its
//     accumulator in place.  A 64-column block per wave keeps the nibble
//     unpacking (VALU) at four weight fragments per step.
//   * Tiles are numbered so that each XCD (workgroups are dealt round-robin
//     over 8, and the grid is a multiple of 8) owns a contiguous, M-grouped
//     range of tiles.
// Lane (j, q) covers k = q*32 .. q*32+31 of a step: k-substep t uses
// k = q*32 + t*16 .. +15 for both operands (low / high half of the lane's 16
// packed weight bytes).
// -------------------------------------------------------------------------
constexpr int R3_BK = 128;
constexpr int R3_ASTAGE = BBM * R3_BK;       // 32 KB of codes
constexpr int R3_WSTAGE = BBN * R3_BK / 2;   // 16 KB of packed weights
constexpr int R3_SLOT = R3_ASTAGE + R3_WSTAGE;
constexpr int R3_WAVES = 8;
constexpr int R3_ALOADS = R3_ASTAGE / 1024 / R3_WAVES;  // 1 KB per load: 4 per wave
constexpr int R3_WLOADS = R3_WSTAGE / 1024 / R3_WAVES;  // 2 per wave
constexpr int R3_EPR = 68;  // epilogue strip row in words (64 + 4 pad)
static_assert(R3_WAVES * 16 * R3_EPR * 4 + 2 * BBN * 4 + BBM * 4 <= R3_SLOT, "epilogue must fit in one slot");

__device__ __forceinline__ v4i r3_half(v4u p, int t)
{
    uint32_t a, b, c, d;
    unpack16(t ? p.z : p.x, a, b);
    unpack16(t ? p.w : p.y, c, d);
    return (v4i){(int)a, (int)b, (int)c, (int)d};
}

// chunk permutation of code row r in LDS (depends on bits 1 and 2 of r)
__device__ __forceinline__ int r3_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 1); }

struct R3Tile {
    int64_t m0, n0;
    __amdgpu_buffer_rsrc_t ra, rw;
};

__device__ __forceinline__ R3Tile r3_tile(const GemmArgs& a, int t, int ntiles, int tiles_n)
{
    R3Tile r;
    if (t >= ntiles) {  // no such tile: zero-sized buffers, every load reads zero
        r.m0 = 0; r.n0 = 0;
        r.ra = make_rsrc(a.codes, 0);
        r.rw = make_rsrc(a.wp, 0);
        return r;
    }
    const int q8 = ntiles >> 3, r8 = ntiles & 7;
    const int xcd = t & 7, loc = t >> 3;
    const int tile = xcd * q8 + min(xcd, r8) + loc;
    constexpr int GROUP_M = 8;
    const int tiles_m = ntiles / tiles_n;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile - (tile / per_group) * per_group;
    r.m0 = (int64_t)(first_m + in_g % gsize) * BBM;
    r.n0 = (int64_t)(in_g / gsize) * BBN;
    r.ra = make_rsrc(a.codes + r.m0 * a.K, (uint64_t)(a.M - r.m0) * a.K);
    r.rw = make_rsrc(a.wp + r.n0 * (a.K >> 1), (uint64_t)(a.N - r.n0) * (a.K >> 1));
    return r;
}

template <int ODT>
__global__ __launch_bounds__(512) void w4a4_gemm_ring3_kernel(GemmArgs a, int tiles_m, int tiles_n)
{
    __shared__ __align__(16) int8_t smem[3 * R3_SLOT];
    static_assert(R3_ALOADS + R3_WLOADS == 6, "vmcnt immediates below assume 6 loads per stage");

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;  // 128-row block wm, 64-column block wn

    const int ntiles = tiles_m * tiles_n;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int nsteps = (int)(K / R3_BK);
    int t = blockIdx.x;
    const int G = gridDim.x;

    // codes: wave w fills tile rows w*32 .. w*32+31, eight rows per load;
    // lane l writes chunk (l & 7) of row (l >> 3), i.e. logical chunk
    // (l & 7) ^ r3_swz(row) (the row's low three bits are l >> 3).
    const int a_vo = (int)((lane >> 3) * K + (((lane & 7) ^ r3_swz(lane >> 3)) * 16));
    const int a_row8 = (int)(8 * K);
    // weights: wave w fills tile columns w*32 .. w*32+31, sixteen per load;
    // lane l writes chunk (l & 3) of column (l >> 2).
    const int w_vo = (int)((wave * 32 + (lane >> 2)) * (K >> 1) + (((lane & 3) ^ ((lane >> 3) & 3)) * 16));
    const int w_col16 = (int)(16 * (K >> 1));
    auto issue = [&](int slot, const __amdgpu_buffer_rsrc_t& ra, const __amdgpu_buffer_rsrc_t& rw, int st) {
        int8_t* as = smem + slot * R3_SLOT;
        int8_t* ws = as + R3_ASTAGE;
        const int ka = st * R3_BK, kw = st * (R3_BK / 2);
#pragma unroll
        for (int i = 0; i < R3_ALOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(as + (wave * 32 + i * 8) * R3_BK), 16,
                a_vo + (wave * 4 + i) * a_row8 + ka, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < R3_WLOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(ws + (wave * 32 + i * 16) * (R3_BK / 2)), 16,
                w_vo + i * w_col16 + kw, 0, 0, 0);
    };

    v4i acc[8][4];
    // fragment offsets inside a slot
    const int w_ro = R3_ASTAGE + (wn * 64 + j) * (R3_BK / 2) + ((q ^ ((j >> 1) & 3)) * 16);
    const int a_ro = (wm * 128 + j) * R3_BK;
    const int a_c0 = ((q * 2) ^ r3_swz(j)) * 16, a_c1 = ((q * 2 + 1) ^ r3_swz(j)) * 16;
    // One step: the weight fragments and the code fragments of substep 0,
    // then those of substep 1 while substep 0 multiplies.
    auto compute = [&](int slot) {
        const int8_t* as = smem + slot * R3_SLOT + a_ro;
        const int8_t* ws = smem + slot * R3_SLOT + w_ro;
        v4u wp[4];
        v4i af[2][8];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) wp[nt] = *(const v4u*)(ws + nt * 16 * (R3_BK / 2));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                af[tt][mt] = *(const v4i*)(as + mt * 16 * R3_BK + (tt ? a_c1 : a_c0));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const v4i bf = r3_half(wp[nt], tt);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tt][mt], bf, acc[mt][nt], 0, 0, 0);
            }
    };

    R3Tile cur_t = r3_tile(a, t, ntiles, tiles_n);
    R3Tile nxt_t = r3_tile(a, t + G, ntiles, tiles_n);
    // Loads are issued unconditionally: stages past the end of a tile belong
    // to the next tile (or read zeros when there is none), so the loop carries
    // no control flow around them.
    issue(0, cur_t.ra, cur_t.rw, 0);
    issue(1, cur_t.ra, cur_t.rw, 1);
    int cur = 0, nxt2 = 2;
    for (;;) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};
        for (int s = 0; s < nsteps; ++s) {
            __builtin_amdgcn_s_waitcnt(0x0f76);  // vmcnt(6): stage s has landed
            __builtin_amdgcn_s_barrier();
            const bool same = s + 2 < nsteps;
            issue(nxt2, same ? cur_t.ra : nxt_t.ra, same ? cur_t.rw : nxt_t.rw,
                  same ? s + 2 : s + 2 - nsteps);
            __builtin_amdgcn_sched_barrier(0);
            compute(cur);
            cur = cur == 2 ? 0 : cur + 1;
            nxt2 = nxt2 == 2 ? 0 : nxt2 + 1;
        }

        // ---- epilogue in the slot the last step used (every wave has left it
        // after the barrier below); the next tile's first two stages are
        // already in flight into the other two.  Scales and bias are widened
        // in LDS; each wave passes its accumulators through LDS as 16 x 64
        // strips so that every store instruction writes whole output rows.
        int8_t* eslot = smem + nxt2 * R3_SLOT;  // == slot of the step just computed
        __builtin_amdgcn_s_barrier();
        float* scol = (float*)(eslot + R3_WAVES * 16 * R3_EPR * 4);
        float* bcol = scol + BBN;
        float* srow = bcol + BBN;
        const int64_t m0 = cur_t.m0, n0 = cur_t.n0;
        {
            // one round trip per tile for the column scales, the bias and the
            // row scales
            const int c = tid & (BBN - 1);
            const int64_t col = n0 + c, row = m0 + c;
            const int64_t cc = col < N ? col : N - 1;
            if (tid < BBN) {
                scol[c] = load_any_f32(a.sw_dtype, a.sw, cc);
                srow[c] = a.sa[row < M ? row : M - 1];
            } else {
                bcol[c] = a.bias ? load_any_f32(a.bias_dtype, a.bias, cc) : 0.0f;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS writes done
        __builtin_amdgcn_s_barrier();
        int* strip = (int*)eslot + wave * 16 * R3_EPR;
        // store mapping: each store instruction writes whole rows of the
        // 16 x 64 strip (128 bytes for 16-bit outputs, 256 for fp32): VPR
        // outputs per lane and store, LPR lanes per row, RPI rows per store
        constexpr int VPR = ODT == F32 ? 4 : 8;
        constexpr int LPR = 64 / VPR;
        constexpr int RPI = 64 / LPR;
        const int sr = lane / LPR;            // first strip row of this lane
        const int cb = (lane % LPR) * VPR;    // column offset inside the 64
        const int64_t col0 = n0 + wn * 64 + cb;
        const bool has_bias = a.bias != nullptr;
        // a full tile with 16-byte aligned rows stores with no per-lane checks
        const bool full = m0 + BBM <= M && n0 + BBN <= N && (N % 8) == 0;
        const float* scl = scol + wn * 64 + cb;
        const float* bia = bcol + wn * 64 + cb;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) strip[(4 * q + r) * R3_EPR + nt * 16 + j] = acc[mt][nt][r] >> 4;
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            int iv[16 / RPI][VPR];
#pragma unroll
            for (int i = 0; i < 16 / RPI; ++i)
#pragma unroll
                for (int c4 = 0; c4 < VPR / 4; ++c4) {
                    const int4 v = *(const int4*)(strip + (sr + i * RPI) * R3_EPR + cb + 4 * c4);
                    iv[i][4 * c4] = v.x; iv[i][4 * c4 + 1] = v.y; iv[i][4 * c4 + 2] = v.z; iv[i][4 * c4 + 3] = v.w;
                }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 16 / RPI; ++i) {
                const int tr = wm * 128 + mt * 16 + sr + i * RPI;  // row inside the tile
                const int64_t row = m0 + tr;
                const float sa = srow[tr];
                float o[VPR];
#pragma unroll
                for (int c = 0; c < VPR; ++c) {
                    const float tv = mul_rn(mul_rn((float)iv[i][c], sa), scl[c]);
                    const float tb = add_rn(tv, bia[c]);
                    o[c] = has_bias ? tb : tv;
                }
                if constexpr (ODT == F32) {
                    float* dst = (float*)a.out + row * N + col0;
                    if (full) {
                        *(float4*)dst = make_float4(o[0], o[1], o[2], o[3]);
                    } else if (row < M) {
#pragma unroll
                        for (int c = 0; c < VPR; ++c)
                            if (col0 + c < N) dst[c] = o[c];
                    }
                } else {
                    uint16_t* dst = (uint16_t*)a.out + row * N + col0;
                    uint32_t pk[4];
#pragma unroll
                    for (int c2 = 0; c2 < 4; ++c2)
                        pk[c2] = (uint32_t)f32_to_h<ODT>(o[2 * c2]) |
                                 ((uint32_t)f32_to_h<ODT>(o[2 * c2 + 1]) << 16);
                    if (full) {
                        *(uint4*)dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                    } else if (row < M) {
                        if (col0 + VPR <= N && (N % 8) == 0) {
                            *(uint4*)dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                        } else {
#pragma unroll
                            for (int c = 0; c < VPR; ++c)
                                if (col0 + c < N) dst[c] = (uint16_t)(pk[c >> 1] >> (16 * (c & 1)));
                        }
                    }
                }
            }
        }
        t += G;
        if (t >= ntiles) break;
        cur_t = nxt_t;
        nxt_t = r3_tile(a, t + G, ntiles, tiles_n);
        // the output stores are counted by vmcnt ahead of nothing the next
        // step needs, but the first wait below counts only loads: drain them
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
}

__global__ void fill_zero_i64(int64_t* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

__global__ void split_epilogue_kernel(GemmArgs a)
{
    const int64_t total = a.M * a.N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / a.N, col = i - row * a.N;
        const int64_t v = a.acc64[i];
        if (a.acc_out) a.acc_out[i] = (int32_t)v;  // meaningful while |acc| < 2^31
        float t = (float)v;                        // nearest-even for |v| >= 2^24
        t = mul_rn(t, a.sa[row]);
        t = mul_rn(t, load_any_f32(a.sw_dtype, a.sw, col));
        t = epilogue_tail(t, a, row, col);
        store_any(a.out_dtype, a.out, i, t);
    }
}
// -------------------------------------------------------------------------
// Skinny-M kernel (M <= 64, per-channel weight scales, no K-chunks): the
// packed-weight stream is the whole cost, so the grid is one 1024-thread
// workgroup per 16 output columns and its 16 waves split the K steps of 64
// (wave w takes steps w, w + 16, ...).  A wave issues the code and weight
// loads of up to SK_MAXS steps at once, straight into registers (buffer loads:
// rows past M and columns past N read zeros), then multiplies them with
// v_mfma_i32_16x16x64_i8 (weights unpacked as 16*w).  The 16 partial tiles
// are summed in LDS as exact integers; one thread per output applies the
// epilogue.
// -------------------------------------------------------------------------
constexpr int SK_WAVES = 16;
constexpr int SK_MAXS = 4;    // K steps per wave in flight at once
constexpr int SK_LD = 20;     // LDS row stride of a partial tile, in words

template <int MT>
__global__ __launch_bounds__(1024) void w4a4_gemm_skinny_kernel(GemmArgs a)
{
    __shared__ int32_t part[SK_WAVES][MT * 16 * SK_LD];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, kq = lane >> 4;
    const int64_t M = a.M, K = a.K, N = a.N;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int nsteps = (int)(K / 64);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes, (uint64_t)M * K);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wp + n0 * (K >> 1), (uint64_t)(N - n0) * (K >> 1));
    // lane (j, kq): code row mt*16 + j, bytes kq*16 .. +15 of a step; weight
    // column n0 + j, packed bytes kq*8 .. +7 of a step
    const int a_off = (int)(j * K + kq * 16);
    const int w_off = (int)(j * (K >> 1) + kq * 8);

    v4i acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (v4i){0, 0, 0, 0};
    for (int s0 = wave; s0 < nsteps; s0 += SK_WAVES * SK_MAXS) {
        v4u af[SK_MAXS][MT];
        v2u wf[SK_MAXS];
#pragma unroll
        for (int i = 0; i < SK_MAXS; ++i) {
            const int st = s0 + i * SK_WAVES;
            const int k0 = st * 64;
            if (st < nsteps) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    af[i][mt] = __builtin_amdgcn_raw_buffer_load_b128(rc, a_off + (int)(mt * 16 * K) + k0, 0, 0);
                wf[i] = __builtin_amdgcn_raw_buffer_load_b64(rw, w_off + (k0 >> 1), 0, 0);
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) af[i][mt] = (v4u){0u, 0u, 0u, 0u};
                wf[i] = (v2u){0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < SK_MAXS; ++i) {
            uint32_t b0, b1, b2, b3;
            unpack16(wf[i].x, b0, b1);
            unpack16(wf[i].y, b2, b3);
            const v4i bf = (v4i){(int)b0, (int)b1, (int)b2, (int)b3};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, af[i][mt]), bf, acc[mt], 0, 0, 0);
        }
    }
    // lane (j, kq) holds rows 4 kq + r, column j of each 16 x 16 tile
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][(mt * 16 + 4 * kq + r) * SK_LD + j] = acc[mt][r];
    __syncthreads();
    if (tid < MT * 16 * 16) {
        const int m = tid >> 4, n = tid & 15;
        int32_t sum = 0;
#pragma unroll
        for (int w = 0; w < SK_WAVES; ++w) sum += part[w][m * SK_LD + n];
        const int64_t row = m, col = n0 + n;
        if (row < M && col < N) {
            const int32_t iv = sum >> 4;
            if (a.acc_out) a.acc_out[row * N + col] = iv;
            float t = mul_rn((float)iv, a.sa[row]);
            t = mul_rn(t, load_any_f32(a.sw_dtype, a.sw, col));
            t = epilogue_tail(t, a, row, col);
            store_any(a.out_dtype, a.out, row * N + col, t);
        }
    }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st)
{
    const bool aligned = (a.K % 32) == 0 && ((uintptr_t)a.codes % 16) == 0 &&
                         ((uintptr_t)a.wp % 16) == 0;
    const bool group = a.sw_group > 0;
    // decode-sized M: the skinny kernel (every epilogue variant but group
    // scales and K-chunks)
    if (!group && a.k_chunk == 0 && a.M >= 1 && a.M <= 64 && (a.K % 64) == 0 &&
        ((uintptr_t)a.codes % 16) == 0 && ((uintptr_t)a.wp % 8) == 0) {
        const unsigned gx = (unsigned)((a.N + 15) / 16);
        if (a.M <= 16)
            hipLaunchKernelGGL(w4a4_gemm_skinny_kernel<1>, dim3(gx), dim3(1024), 0, st, a);
        else if (a.M <= 32)
            hipLaunchKernelGGL(w4a4_gemm_skinny_kernel<2>, dim3(gx), dim3(1024), 0, st, a);
        else
            hipLaunchKernelGGL(w4a4_gemm_skinny_kernel<4>, dim3(gx), dim3(1024), 0, st, a);
        return hipGetLastError();
    }
    // Prefill-sized layers take the 256 x 256 three-stage kernel; everything
    // else (small M, group scales, low-rank term, INT32 export, K chunks,
    // K not a multiple of 128, unaligned operands) the 128 x 128 kernel.
    const bool ring3 = !group && a.lora == nullptr && a.acc_out == nullptr && a.k_chunk == 0 &&
                       a.M > 128 && (a.K % R3_BK) == 0 && a.K >= 2 * R3_BK && aligned &&
                       ((uintptr_t)a.out % 16) == 0;
    if (ring3) {
        const int tm = (int)((a.M + BBM - 1) / BBM), tn = (int)((a.N + BBN - 1) / BBN);
        const int nt = tm * tn;
        // persistent grid: one workgroup per CU (a multiple of 8 so that a
        // workgroup's tiles all fall in its XCD), or one per tile if fewer
        static int n_cu = 0;
        if (n_cu == 0) {
            int dev = 0, v = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v >= 8)
                n_cu = v & ~7;
            else
                n_cu = 256;
        }
        const unsigned grid = (unsigned)(nt < n_cu ? nt : n_cu);
        if (a.out_dtype == F32)
            hipLaunchKernelGGL(w4a4_gemm_ring3_kernel<F32>, dim3(grid), dim3(512), 0, st, a, tm, tn);
        else if (a.out_dtype == F16)
            hipLaunchKernelGGL(w4a4_gemm_ring3_kernel<F16>, dim3(grid), dim3(512), 0, st, a, tm, tn);
        else
            hipLaunchKernelGGL(w4a4_gemm_ring3_kernel<BF16>, dim3(grid), dim3(512), 0, st, a, tm, tn);
        return hipGetLastError();
    }
    const unsigned gx = (unsigned)((a.N + BN - 1) / BN);
    const unsigned gy = (unsigned)((a.M + BM - 1) / BM);
    if (a.k_chunk > 0 && !group) {
        const int64_t kc = a.k_chunk;
        const unsigned gz = (unsigned)((a.K + kc - 1) / kc);
        const int64_t n = a.M * a.N;
        hipLaunchKernelGGL(fill_zero_i64, dim3(1024), dim3(256), 0, st, a.acc64, n);
        if (aligned)
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, true, true>), dim3(gx, gy, gz), dim3(256), 0,
                               st, a, kc);
        else
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, true, false>), dim3(gx, gy, gz), dim3(256), 0,
                               st, a, kc);
        hipLaunchKernelGGL(split_epilogue_kernel, dim3(2048), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    const int64_t kc = a.K;
    // (the aligned kernels without K-chunks stage through buffer loads that
    // need whole 64-deep K steps and 32-bit offsets within a 128-row tile)
    const bool aligned_buf = aligned && (a.K % 64) == 0 && a.K <= (1 << 24);
    if (group) {
#define W4A4_GROUP_LAUNCH(DT)                                                                    \
    do {                                                                                         \
        if (aligned_buf)                                                                         \
            hipLaunchKernelGGL((w4a4_gemm_kernel<DT, false, true>), dim3(gx, gy, 1), dim3(256), 0, \
                               st, a, kc);                                                       \
        else                                                                                     \
            hipLaunchKernelGGL((w4a4_gemm_kernel<DT, false, false>), dim3(gx, gy, 1), dim3(256), \
                               0, st, a, kc);                                                    \
    } while (0)
        if (a.sw_dtype == F32) W4A4_GROUP_LAUNCH(F32);
        else if (a.sw_dtype == F16) W4A4_GROUP_LAUNCH(F16);
        else W4A4_GROUP_LAUNCH(BF16);
#undef W4A4_GROUP_LAUNCH
    } else {
        if (aligned_buf)
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, false, true>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
        else
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, false, false>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
    }
    return hipGetLastError();
}

}  // namespace w4a4

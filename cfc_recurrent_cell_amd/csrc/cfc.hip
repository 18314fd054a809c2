// cfc.hip -- gfx950 kernels and the C ABI of libcfc_amd (see include/cfc.h).
//
// Kernels
//   cfc_fwd_small_kernel / cfc_bwd_small_kernel   n_in, n_hid <= 128: one
//       workgroup per batch row runs the whole (reverse) K-loop; dense
//       contractions on the f64 matrix cores, the serial chain on the vector
//       units with W_rec held in registers.  cfc_fb_small_kernel runs both
//       directions in one launch, keeping the forward's a_k on chip.
//   cfc_fwd_large_kernel / cfc_bwd_large_kernel   n_in or n_hid in (128, 256]:
//       a workgroup owns 16 batch rows, so every step is a matrix-core product.
//   cfc_bwd_kernel    general backward (any n_in, n_hid <= 256, and the
//       accumulate mode at the larger sizes when the caller gives no
//       workspace): one workgroup per row, matvecs on the vector units with
//       the weights read from L2.
//   Every backward keeps dL/da for all steps on chip (or parked in its own
//   scratch row, or in the caller's workspace) and forms the weight gradients
//   as contractions over k, so each scratch element is written once (no
//   per-step read-modify-write).
//   reduce_axis0_kernel  column-tiled sum over the leading axis;
//   reduce_rows_narrow_kernel + reduce_partials_kernel  the two-phase sum for
//       narrow rows over a long leading axis.
//
// The block-per-batch layout and the single-writer scratch come from the
// "K-loop Parallelization Implementation Plan" (foxhunt, 2026-05-17), Tasks 2
// and 3; the column-tiled reducer with a padded LDS tree from the ml-alpha
// commit "NVIDIA-grade rewrite of CfC K-loop hot kernels" (b23f8f2efa).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "cfc.h"

namespace {

constexpr int kThreads = 256;             // 4 wave64 per workgroup
constexpr int kMaxIn = CFC_MAX_N_IN;
constexpr int kMaxHid = CFC_MAX_N_HID;
constexpr size_t kLdsBytes = 160 * 1024;  // gfx950 LDS per workgroup

// ------------------------------------------------------------------ math
__device__ __forceinline__ double softplus_f64(double w) {
    // log(1 + e^w) without overflow
    return log1p(exp(-fabs(w))) + fmax(w, 0.0);
}
__device__ __forceinline__ double logistic_f64(double z) { return 1.0 / (1.0 + exp(-z)); }

// The tau-decay cell ("K-loop Parallelization Implementation Plan", Tasks 2
// and 3): a unit's gate is the constant decay = exp(-dt / max(tau, 1e-6)), and
// d decay / d tau = decay * q with q = dt / tau^2 where tau > 1e-6, else 0
// (the pages' zero-gradient guard).
constexpr double kTauEps = 1e-6;
__device__ __forceinline__ void tau_decay_consts(double tau, double dt, double& decay, double& q) {
    const double tau_eff = fmax(tau, kTauEps);
    decay = exp(-dt / tau_eff);
    q = tau > kTauEps ? dt / (tau_eff * tau_eff) : 0.0;
}

// Threads per output of a matvec: the largest power of two G <= 64 with
// G * rows <= 256, so a group of G consecutive lanes shares one output and
// combines with butterfly shuffles inside one wavefront.
__device__ __forceinline__ int group_size(int rows) {
    int g = 1;
    while (g < 64 && 2 * g * rows <= kThreads) g <<= 1;
    return g;
}

// Sum over the G consecutive lanes of a group (every lane of the wave takes
// part, so the shuffles are non-divergent).
__device__ __forceinline__ double group_sum(double v, int G) {
    for (int off = G >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// ----------------------------------------------------------- backward
// The steps one backward launch covers: steps k0 .. k0 + Kw - 1 of a K-step
// forward (row b's x_k at x + (b K + k) n_in, h_k+1 at h_seq + (b K + k) H,
// h_0 in h0).  The gradient flowing into the window's last state h_k0+Kw is
// delta_in [B, H], or, when delta_in is NULL (then k0 + Kw == K), the loss
// seed h_K - y.  delta_out [B, H] (may be NULL; may be delta_in itself, since
// each element is read before the one writer of that element writes it)
// receives dL/dh_k0 -- dL/dh_0 for the first window.  Kernels index steps
// relative to k0.
struct BwdWindow {
    int K, k0, Kw;
    const float* delta_in;
    float* delta_out;
};

// LDS: DA [Kw][H] f64 | delta [2][H] f64 | gate [H] f64 | sp [H] | sw [H] |
//      red [256] f64 | xs [Kw][n_in] f32 | hp [Kw][H] f32   (hp[k] = h_k0+k)
__host__ __device__ inline size_t bwd_lds_bytes(int K, int n_in, int H) {
    return (size_t)8 * K * H + (size_t)8 * 5 * H + 8 * kThreads + (size_t)4 * K * n_in +
           (size_t)4 * K * H;
}

// Accumulate mode adds this call's gradient, rounded to float32, to the stored
// value in float32 (a float32 += into the scratch), in every kernel.
__device__ __forceinline__ void store_grad(float* p, double v, int accumulate) {
    *p = accumulate ? (float)v + *p : (float)v;
}

__global__ __launch_bounds__(kThreads) void cfc_bwd_kernel(
    const float* __restrict__ w_in, const float* __restrict__ w_rec,
    const float* __restrict__ bias, const float* __restrict__ w_tau,
    const float* __restrict__ x, const float* __restrict__ h0, const float* __restrict__ h_seq,
    const float* __restrict__ y, double dt, BwdWindow win, int n_in, int H, float* __restrict__ scratch,
    float* __restrict__ loss, float* __restrict__ grad_x, int accumulate, int cell) {
    const int K = win.Kw;  // steps of this launch; indices below are relative to win.k0
    const long long Kf = win.K, k0 = win.k0;
    extern __shared__ __align__(16) unsigned char smem[];
    double* DA = reinterpret_cast<double*>(smem);
    double* delta = DA + (size_t)K * H;
    double* gate = delta + 2 * H;
    double* sp = gate + H;
    double* sw = sp + H;
    double* red = sw + H;
    float* xs = reinterpret_cast<float*>(red + kThreads);
    float* hp = xs + (size_t)K * n_in;

    const int t = threadIdx.x;
    const long long b = blockIdx.x;
    const long long N = (long long)H * (n_in + H + 2);
    const int G = group_size(H);
    const int i = t / G, sub = t % G;

    // per-unit constants, staged row inputs, loss seed
    double lpart = 0.0;
    for (int u = t; u < H; u += kThreads) {
        const double w = (double)w_tau[u];
        if (cell == CFC_CELL_TAU_DECAY) {
            tau_decay_consts(w, dt, sp[u], sw[u]);  // sp = decay, sw = d decay / d tau / decay
        } else {
            sp[u] = softplus_f64(w);
            sw[u] = logistic_f64(w);
        }
        if (win.delta_in) {
            delta[u] = (double)win.delta_in[b * H + u];
        } else {
            const double d = (double)h_seq[(b * Kf + (Kf - 1)) * H + u] - (double)y[b * H + u];
            delta[u] = d;
            lpart += 0.5 * d * d;
        }
    }
    const float* xb = x + (b * Kf + k0) * n_in;
    for (int e = t; e < K * n_in; e += kThreads) xs[e] = xb[e];
    const float* hstart = k0 == 0 ? h0 + b * H : h_seq + (b * Kf + k0 - 1) * H;
    for (int u = t; u < H; u += kThreads) hp[u] = hstart[u];
    const float* hsb = h_seq + (b * Kf + k0) * H;
    for (int e = t; e < (K - 1) * H; e += kThreads) hp[H + e] = hsb[e];
    red[t] = lpart;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (t < s) red[t] += red[t + s];
        __syncthreads();
    }
    if (t == 0 && loss) loss[b] = (float)red[0];

    // serial reverse chain: dL/da_k for every k, delta carried through W_rec^T
    double gb = 0.0, gwt = 0.0;  // owned by the lane with sub == 0 of unit i
    int cur = 0;
    for (int k = K - 1; k >= 0; --k) {
        const float* xk = xs + k * n_in;
        const float* hk = hp + k * H;
        double part = 0.0;
        if (i < H) {
            const float* wi = w_in + (long long)i * n_in;
            const float* wr = w_rec + (long long)i * H;
            for (int j = sub; j < n_in; j += G) part = fma((double)wi[j], (double)xk[j], part);
            for (int j = sub; j < H; j += G) part = fma((double)wr[j], (double)hk[j], part);
        }
        part = group_sum(part, G);
        if (i < H && sub == 0) {
            const double a = (double)bias[i] + part;
            const double c = tanh(a);
            const double d = delta[cur * H + i];
            double g, da;
            if (cell == CFC_CELL_TAU_DECAY) {
                g = sp[i];
                const double dg = d * ((double)hk[i] - c);  // dL/d(decay)
                da = d * (1.0 - g) * (1.0 - c * c);
                gwt += dg * g * sw[i];
            } else {
                g = 1.0 / (1.0 + exp(sp[i] * a * dt));
                const double dz = d * ((double)hk[i] - c) * g * (1.0 - g);
                da = d * (1.0 - g) * (1.0 - c * c) - dz * sp[i] * dt;
                gwt += dz * (-a * dt) * sw[i];
            }
            DA[k * H + i] = da;
            gate[i] = g;
            gb += da;
        }
        __syncthreads();
        // delta_k = delta_{k+1} * g + W_rec^T da ; here i indexes the column j
        double p2 = 0.0;
        if (i < H) {
            const double* dak = DA + k * H;
            for (int r = sub; r < H; r += G) p2 = fma((double)w_rec[(long long)r * H + i], dak[r], p2);
        }
        p2 = group_sum(p2, G);
        if (i < H && sub == 0) delta[(cur ^ 1) * H + i] = delta[cur * H + i] * gate[i] + p2;
        cur ^= 1;
        __syncthreads();
    }

    // weight gradients as contractions over k; one store per scratch element
    float* row = scratch + b * N;
    for (int e = t; e < H * n_in; e += kThreads) {
        const int r = e / n_in, j = e - r * n_in;
        double s = 0.0;
        for (int k = 0; k < K; ++k) s = fma(DA[k * H + r], (double)xs[k * n_in + j], s);
        store_grad(row + e, s, accumulate);
    }
    float* rrec = row + (long long)H * n_in;
    for (int e = t; e < H * H; e += kThreads) {
        const int r = e / H, j = e - r * H;
        double s = 0.0;
        for (int k = 0; k < K; ++k) s = fma(DA[k * H + r], (double)hp[k * H + j], s);
        store_grad(rrec + e, s, accumulate);
    }
    if (i < H && sub == 0) {
        store_grad(rrec + (long long)H * H + i, gb, accumulate);
        store_grad(rrec + (long long)H * H + H + i, gwt, accumulate);
    }
    // input gradients: dL/dh_k0 is the delta left after the window's first
    // step; dL/dx_k = W_in^T da_k
    if (win.delta_out)
        for (int u = t; u < H; u += kThreads) win.delta_out[b * H + u] = (float)delta[cur * H + u];
    if (grad_x) {
        float* gx = grad_x + (b * Kf + k0) * n_in;
        for (int e = t; e < K * n_in; e += kThreads) {
            const int k = e / n_in, j = e - k * n_in;
            double s = 0.0;
            for (int r = 0; r < H; ++r) s = fma(DA[k * H + r], (double)w_in[(long long)r * n_in + j], s);
            gx[e] = (float)s;
        }
    }
}

// =====================================================================
// Kernels for n_in <= 128 and n_hid <= 128 (the smoke and training-scale
// workloads): every dimension is zero-padded to 128 inside the kernel, which
// leaves the results unchanged (padded units keep a = 0, h = 0, delta = 0).
//
// One workgroup of 4 wave64 per batch row, as above, but
//  * the three dense contractions -- the input projection U = X W_in^T + b
//    (forward), the recomputed pre-activations A = [X | H_prev] [W_in | W_rec]^T
//    + b (backward) and the weight gradients DA^T [X | H_prev] (backward) --
//    run on the f64 matrix cores (v_mfma_f64_16x16x4f64); the weight operand
//    of the first two is held in registers for the whole contraction;
//  * the serial chain keeps W_rec (or W_rec^T) in registers, an 8x8 slice per
//    lane: lane (ib, jb) holds rows 8ib..8ib+7, columns 8jb..8jb+7, reads 8
//    values of the state from LDS per step, and the 16 lanes of a row block
//    combine with a DPP reduce-scatter so that lanes jb and jb^1 both end with
//    the total of one output unit (ChainLane below);
//  * those two lanes share the transcendental work: one evaluates
//    exp(2a) -> tanh(a) = 1 - 2/(1+exp(2a)), the other exp(sp a dt) -> the gate
//    1/(1+exp(sp a dt)), and they swap results.
// =====================================================================
typedef double dbl4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// D(16x16) += A(16x4) B(4x16) in f64.  Lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; element v of lane l is D[l/16 + 4v][l%16] (checked on gfx950).
__device__ __forceinline__ dbl4 mfma_f64(double a, double b, dbl4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// DPP lane moves: quad_perm xor 1 (0xB1), quad_perm xor 2 (0x4E), and
// row_half_mirror (0x141: lane i of each 8-lane half-row reads lane 7 - i).
template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
    // two 32-bit DPP moves; every lane of the patterns used here has a valid
    // source, so no fallback value is needed
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141;

constexpr int kDppRor8 = 0x128;  // row_ror:8: lane i of each 16-lane row reads lane i ^ 8

// Sum of v over the 64 lanes of the wave, in every lane: within each 16-lane
// row by DPP (xor 1, xor 2, half-mirror, ror 8), then the four row sums read
// out by lane.  A fixed order, and no LDS round trips.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_move<kDppXor1>(v);
    v += dpp_move<kDppXor2>(v);
    v += dpp_move<kDppHalfMirror>(v);
    v += dpp_move<kDppRor8>(v);
    auto lane_value = [](double x, int l) {
        const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
        const unsigned lo = __builtin_amdgcn_readlane((int)(unsigned)u, l);
        const unsigned hi = __builtin_amdgcn_readlane((int)(unsigned)(u >> 32), l);
        return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
    };
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Serial-chain layout of the one-row kernels.  Lane (wave w, row r = lane / 16,
// l = lane % 16) owns unit o = 32w + 16 (r / 2) + l over the column half
// hf = r % 2 (columns 64hf .. 64hf + 63 of the step's 128 x 128 product), so
// rows 2p and 2p + 1 of a wave hold the same 16 units over the two halves.  A
// lane keeps the 64 weights of its unit and half in registers and reads 4
// values of the state (columns 64hf + 4l .. 64hf + 4l + 3) from LDS per step;
// the 16 lanes of a row broadcast their state values to each other inside the
// product (v_fmac_f64 with row_newbcast DPP: lane j's value multiplies every
// lane's own weight), so the product needs no reduction inside the row.  The
// two halves are added across the row pair with v_permlane16_swap, which leaves
// the same sum, bitwise, in both lanes of the unit; the even-row lane then
// evaluates tanh and the odd-row lane the gate.
struct ChainLane {
    int o, hf, l;
    bool gate;
};
__device__ __forceinline__ ChainLane chain_lane(int wave, int lane) {
    const int r = lane >> 4, l = lane & 15;
    return ChainLane{32 * wave + 16 * (r >> 1) + l, r & 1, l, (r & 1) != 0};
}

// Both lanes of a row pair get the even row's v and the odd row's v (the two
// 32-bit halves go through v_permlane16_swap, which exchanges a register's odd
// rows with another's even rows).
__device__ __forceinline__ void row_pair_values(double v, double& even, double& odd) {
    // the swap overwrites both of its operands: a second copy of v, made by
    // one 64-bit move (the empty asm keeps it a distinct register), instead
    // of a 32-bit move per half
    double w = v;
    asm volatile("" : "+v"(w));
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const unsigned long long uw = __builtin_bit_cast(unsigned long long, w);
    const auto lo = __builtin_amdgcn_permlane16_swap((unsigned)u, (unsigned)uw, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(u >> 32), (unsigned)(uw >> 32), false, false);
    even = __builtin_bit_cast(double, ((unsigned long long)hi[0] << 32) | lo[0]);
    odd = __builtin_bit_cast(double, ((unsigned long long)hi[1] << 32) | lo[1]);
}

// The lane's 4 state values of columns 64hf + 4l .. 64hf + 4l + 3 (two 16-byte
// LDS reads; a row reads 512 contiguous bytes).
__device__ __forceinline__ void chain_read(double (&s)[4], const double* v, const ChainLane& cl) {
    const double2* p = reinterpret_cast<const double2*>(v + 64 * cl.hf + 4 * cl.l);
    const double2 v0 = p[0], v1 = p[1];
    s[0] = v0.x;
    s[1] = v0.y;
    s[2] = v1.x;
    s[3] = v1.y;
}

// seed + sum over j < 16, m < 4 of w[j][m] * (lane j's s[m]) for this lane's
// half of the unit, in a fixed order into two accumulators (both seeded with
// `seed`): 64 v_fmac_f64 whose first operand is broadcast from lane j of the
// row (row_newbcast:j).  Two asm statements, one per pair of state values, so
// that the first can start when the first LDS read has returned.  Each begins
// with two wait states, the distance a DPP source needs from a vector-ALU write
// of it.
#define CFC_FMAC_J(J, S, W)                                                                  \
    "v_fmac_f64_dpp %[a0], %[" #S "a], %[" #W "0_" #J "] row_newbcast:" #J " row_mask:0xf bank_mask:0xf\n" \
    "v_fmac_f64_dpp %[a1], %[" #S "b], %[" #W "1_" #J "] row_newbcast:" #J " row_mask:0xf bank_mask:0xf\n"
#define CFC_FMAC_16(S, W)                                                                    \
    CFC_FMAC_J(0, S, W) CFC_FMAC_J(1, S, W) CFC_FMAC_J(2, S, W) CFC_FMAC_J(3, S, W)           \
    CFC_FMAC_J(4, S, W) CFC_FMAC_J(5, S, W) CFC_FMAC_J(6, S, W) CFC_FMAC_J(7, S, W)           \
    CFC_FMAC_J(8, S, W) CFC_FMAC_J(9, S, W) CFC_FMAC_J(10, S, W) CFC_FMAC_J(11, S, W)         \
    CFC_FMAC_J(12, S, W) CFC_FMAC_J(13, S, W) CFC_FMAC_J(14, S, W) CFC_FMAC_J(15, S, W)
#define CFC_W_OPS(W, M0, M1)                                                                  \
    [W##0_0] "v"(w[0][M0]), [W##1_0] "v"(w[0][M1]), [W##0_1] "v"(w[1][M0]), [W##1_1] "v"(w[1][M1]),         \
    [W##0_2] "v"(w[2][M0]), [W##1_2] "v"(w[2][M1]), [W##0_3] "v"(w[3][M0]), [W##1_3] "v"(w[3][M1]),         \
    [W##0_4] "v"(w[4][M0]), [W##1_4] "v"(w[4][M1]), [W##0_5] "v"(w[5][M0]), [W##1_5] "v"(w[5][M1]),         \
    [W##0_6] "v"(w[6][M0]), [W##1_6] "v"(w[6][M1]), [W##0_7] "v"(w[7][M0]), [W##1_7] "v"(w[7][M1]),         \
    [W##0_8] "v"(w[8][M0]), [W##1_8] "v"(w[8][M1]), [W##0_9] "v"(w[9][M0]), [W##1_9] "v"(w[9][M1]),         \
    [W##0_10] "v"(w[10][M0]), [W##1_10] "v"(w[10][M1]), [W##0_11] "v"(w[11][M0]), [W##1_11] "v"(w[11][M1]), \
    [W##0_12] "v"(w[12][M0]), [W##1_12] "v"(w[12][M1]), [W##0_13] "v"(w[13][M0]), [W##1_13] "v"(w[13][M1]), \
    [W##0_14] "v"(w[14][M0]), [W##1_14] "v"(w[14][M1]), [W##0_15] "v"(w[15][M0]), [W##1_15] "v"(w[15][M1])
__device__ __forceinline__ double chain_product(const double (&w)[16][4], const double (&s)[4], double seed) {
    double a0 = seed, a1 = seed;
    asm volatile("s_nop 1\n" CFC_FMAC_16(s0, w)
                 : [a0] "+v"(a0), [a1] "+v"(a1)
                 : [s0a] "v"(s[0]), [s0b] "v"(s[1]), CFC_W_OPS(w, 0, 1));
    asm volatile("s_nop 1\n" CFC_FMAC_16(s1, x)
                 : [a0] "+v"(a0), [a1] "+v"(a1)
                 : [s1a] "v"(s[2]), [s1b] "v"(s[3]), CFC_W_OPS(x, 2, 3));
    return a0 + a1;
}
#undef CFC_FMAC_J
#undef CFC_FMAC_16
#undef CFC_W_OPS

// The unit's full sum in both lanes of the row pair: the two halves' partial
// sums added in the order (even row) + (odd row), so both lanes hold the same
// bits.
__device__ __forceinline__ double chain_total(double half_sum) {
    double even, odd;
    row_pair_values(half_sum, even, odd);
    return even + odd;
}

// e^x for |x| <= 700: x = n ln2 + r with n = rint(x log2e) and r by one FMA
// with ln2 rounded to double (the reduction error |n| 2.3e-17 is below
// 1.5e-15 relative for |x| < 40 and below 2.4e-14 at |x| = 700), |r| <= ln2/2,
// e^r by a degree-10 polynomial with constant term 1 whose other coefficients
// minimise the largest relative error on [-ln2/2, ln2/2] (Remez exchange,
// computed in 50-digit arithmetic and rounded to double: 2.4e-15 relative,
// against 2.4e-13 for the degree-10 Taylor polynomial), evaluated with
// Estrin's scheme for a short dependency chain, then scaled by 2^n.
constexpr double kLog2e = 1.4426950408889634074;
constexpr double kLn2 = 0.69314718055994530942;
__device__ __forceinline__ double exp_poly_scaled(double r, int n) {
    constexpr double c1 = 1.0000000000000009, c2 = 0.49999999999997086, c3 = 0.16666666666632235,
                     c4 = 0.04166666667007467, c5 = 0.008333333358760514, c6 = 0.0013888887798236404,
                     c7 = 0.00019841203906994798, c8 = 2.4802862967019124e-05, c9 = 2.7626408481260957e-06,
                     c10 = 2.7086871132720806e-07;
    const double r2 = r * r, r4 = r2 * r2, r8 = r4 * r4;
    auto fma3 = [](double a, double x, double c) {
        double d;
        asm("v_fma_f64 %0, %1, %2, %3" : "=v"(d) : "s"(a), "v"(x), "v"(c));
        return d;
    };
    const double q0 = fma(c1, r, 1.0), q1 = fma3(c3, r, c2), q2 = fma3(c5, r, c4), q3 = fma3(c7, r, c6);
    const double q4 = fma3(c9, r, c8);
    const double s0 = fma(q1, r2, q0), s1 = fma(q3, r2, q2), s2 = fma(c10, r2, q4);
    const double t0 = fma(s1, r4, s0);
    return ldexp(fma(s2, r8, t0), n);
}
// The reduction of both forms below: adding 1.5 * 2^52 to x log2e (one FMA
// from x) rounds it to the nearest integer n, which then sits in the low bits
// of the sum's significand (exact for |x log2e| < 2^51), so n = t - 1.5 * 2^52
// and the integer exponent are read off the sum with no rounding or
// float-to-int instruction.
constexpr double kExpShift = 6755399441055744.0;  // 1.5 * 2^52

// 1 / (1 + e^z) for finite z: |z| is clamped to 700 (beyond it the result is
// 0 or 1 to double precision).  The reciprocal is v_rcp_f64 (24 correct bits,
// measured over a full binade) and one Newton step: about 2e-15 relative.
// The clamp maps a NaN z to a finite value, so this form serves rows whose
// inputs are all finite (then every pre-activation is finite: |a| stays below
// 1e80 for float32 inputs); inv_one_plus_exp_exact serves the others.
__device__ __forceinline__ double inv_one_plus_exp(double z) {
    z = fmin(fmax(z, -700.0), 700.0);
    const double t = fma(z, kLog2e, kExpShift);
    const double n = t - kExpShift;
    const int ni = (int)(unsigned)__builtin_bit_cast(unsigned long long, t);
    const double d = 1.0 + exp_poly_scaled(fma(-n, kLn2, z), ni);
    const double y = __builtin_amdgcn_rcp(d);
    const double e = fma(-d, y, 1.0);
    return fma(y, e, y);
}

// 1 / (1 + e^(m a)) for any a, with m_log2e = m log2e: NaN in, NaN out.
// z = m a and t = fma(m_log2e, a, 1.5 * 2^52) are formed side by side.
// Where |z| > 700 the result is 0 or 1 to double precision and is selected
// after the evaluation (whose value is then unspecified); a NaN z fails that
// comparison and comes out as NaN.
__device__ __forceinline__ double inv_one_plus_exp_exact(double m, double m_log2e, double a) {
    const double z = m * a;
    const double t = fma(m_log2e, a, kExpShift);
    const double n = t - kExpShift;
    const int ni = (int)(unsigned)__builtin_bit_cast(unsigned long long, t);
    const double d = 1.0 + exp_poly_scaled(fma(-n, kLn2, z), ni);
    const double y = __builtin_amdgcn_rcp(d);
    const double e = fma(-d, y, 1.0);
    const double v = fma(y, e, y);
    return fabs(z) > 700.0 ? (z > 0.0 ? 0.0 : 1.0) : v;
}

// The gate of one unit for both cells, as constants of one set of formulas
// (padding units get g = 1/2 and no gradient terms):
//   g                 = vadd + vmul / (1 + e^(zmul a))
//                       (gated: 1/(1+e^(softplus(w_tau) dt a)); tau-decay: decay)
//   dz                = delta (h - c) g (1 - vmul g)
//   dL/da             = delta (1 - g)(1 - c^2) - dz rho
//   dL/dw_tau (dtau) += dz (beta - a alpha)
struct UnitGate {
    double zmul, vmul, vadd, rho, alpha, beta;
};
__device__ __forceinline__ UnitGate unit_gate(int cell, double w, double dt, bool valid) {
    if (!valid) return UnitGate{0.0, 1.0, 0.0, 0.0, 0.0, 0.0};
    if (cell == CFC_CELL_TAU_DECAY) {
        double decay, q;
        tau_decay_consts(w, dt, decay, q);
        return UnitGate{0.0, 0.0, decay, 0.0, 0.0, q};
    }
    const double spdt = softplus_f64(w) * dt;
    return UnitGate{spdt, 1.0, 0.0, spdt, dt * logistic_f64(w), 0.0};
}

// Per-lane constants of cell_gates: the gate lane evaluates the gate above,
// the tanh lane 1 - 2/(1+e^(2a)).
struct GateLane {
    double zmul, vmul, vadd;
    bool gate;
};
__device__ __forceinline__ GateLane gate_lane_consts(bool gate_lane, const UnitGate& u) {
    return GateLane{gate_lane ? u.zmul : 2.0, gate_lane ? u.vmul : -2.0, gate_lane ? u.vadd : 1.0, gate_lane};
}

// tanh(a) and the gate for the unit owned by a lane pair: the even-row lane
// evaluates tanh, the odd-row lane the gate, and the row-pair exchange gives
// both lanes both values.
__device__ __forceinline__ void cell_gates(double a, const GateLane& L, double& g, double& c) {
    const double r = inv_one_plus_exp(L.zmul * a);
    row_pair_values(fma(r, L.vmul, L.vadd), c, g);
}
// The same for a row whose inputs are not all finite: NaN propagates as in the
// definition (zl = L.zmul * log2e, hoisted by the caller).
__device__ __forceinline__ void cell_gates_exact(double a, const GateLane& L, double zl, double& g, double& c) {
    const double r = inv_one_plus_exp_exact(L.zmul, zl, a);
    row_pair_values(fma(r, L.vmul, L.vadd), c, g);
}

// A float4 store of a gradient stream that the reducer reads next from HBM
// (the gigabyte scratch of the wide kernels), with the cache-policy bits
// sc1 nt: written through without leaving dirty lines in the caches.  With
// plain non-temporal stores the reduce that followed the large-batch backward
// paid for writing back the backward's last dirty lines (0.78 ms against
// 0.70 ms on a flushed buffer); with these it takes 0.71 ms, and the backward's
// weight-gradient phase 0.845 instead of 0.87 ms (measured on MI355X; plain
// stores 0.90 and 0.86 ms, sc1 alone 0.89 and 0.86 ms).  The compiler does not
// see the store inside the asm, so the asm ends with two wait states: a vector
// instruction may not overwrite the data registers of a store wider than 8
// bytes right after it.
__device__ __forceinline__ void store_stream_f32x4(float* dst, f32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
}

// s_waitcnt lgkmcnt(0): wait for every outstanding LDS and scalar-memory
// access.  Placed at the top of a chain loop, where the previous step's barrier
// has already drained the LDS queue, it costs nothing; it tells the compiler's
// wait insertion that no scalar load issued before the loop is still in
// flight.  Scalar loads return out of order, so without it the loop's first
// LDS wait (its state read) becomes a wait for all of the step's LDS reads in
// every iteration (measured: the forward chain about 80 cycles per step slower).
__device__ __forceinline__ void lds_and_scalar_drained() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <bool EXACT>
__device__ __forceinline__ void cell_gates_t(double a, const GateLane& L, double zl, double& g, double& c) {
    if constexpr (EXACT)
        cell_gates_exact(a, L, zl, g, c);
    else
        cell_gates(a, L, g, c);
}

// Rows whose chains consume a non-finite value (a NaN or infinity in x, h_0,
// h_seq, the weights, the bias or w_tau reaches the projection, the chain
// weights, the initial state or the gate constants) run the chain loops with
// cell_gates_exact; all others run the shorter cell_gates.  Each thread tests
// what it loaded or computed, and the workgroup ORs the tests through one LDS
// word, so the choice is uniform across the workgroup.
__device__ __forceinline__ bool not_finite(double v) { return !__builtin_isfinite(v); }
__device__ __forceinline__ bool any_not_finite(const UnitGate& u) {
    return not_finite(u.zmul) || not_finite(u.vmul) || not_finite(u.vadd) || not_finite(u.rho) ||
           not_finite(u.alpha) || not_finite(u.beta);
}
template <int R, int C>
__device__ __forceinline__ bool any_not_finite(const double (&w)[R][C]) {
    bool bad = false;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) bad |= not_finite(w[r][c]);
    return bad;
}

constexpr int kSmall = 128;          // padded n_in and n_hid of the small kernels
constexpr int kSmallFwdKW = 64;      // forward steps per window
constexpr int kSmallBwdMaxK = 64;    // backward: whole K-loop on chip
constexpr int kSmallXS = kSmall + 2;             // padded LDS row stride (floats)
constexpr int kSmallZW = 2 * kSmall;             // [x | h_prev] width
constexpr int kSmallZS = kSmallZW + 2;
// Row stride (doubles) of the one-row kernels' a / dL/da array: 4 doubles of
// padding put the 16 rows that one matrix-core operand read touches in
// different LDS banks (with 128 doubles per row they all fell in one).
constexpr int kSmallAS = kSmall + 4;

__host__ __device__ constexpr size_t small_fwd_lds_bytes() {
    return (size_t)8 * kSmallFwdKW * kSmall + (size_t)8 * 2 * kSmall + 16 +
           (size_t)4 * kSmallFwdKW * kSmallXS;
}
// The backward always stages kSmallBwdMaxK rows (rows >= K are zero), so its
// contractions run without row guards.
constexpr int kSmallGS = 64 + 4;  // row stride (floats) of a wave's gradient-tile buffer
__host__ __device__ constexpr size_t small_bwd_lds_bytes() {
    return (size_t)8 * kSmallBwdMaxK * kSmallAS + 8 * 8 +
           (size_t)4 * kSmallBwdMaxK * kSmallZS + (size_t)4 * 4 * 16 * kSmallGS;
}

// Copy `rows` rows of `width` floats (source rows contiguous, row stride
// src_stride) into LDS rows of stride dst_stride, zero-filling columns
// [width, pad_width) and rows [rows, pad_rows).  Vector path when the source is
// 16-byte aligned and width == pad_width is a multiple of 4.
__device__ __forceinline__ void stage_rows(float* dst, int dst_stride, const float* src,
                                           long long src_stride, int rows, int width, int pad_rows,
                                           int pad_width, int t) {
    const bool vec = width == pad_width && (width & 3) == 0 && (src_stride & 3) == 0 &&
                     (reinterpret_cast<uintptr_t>(src) & 15) == 0;
    if (vec) {
        const int q = width >> 2;  // float4 per row
        const int total = pad_rows * q;
        for (int e0 = t; e0 < total; e0 += 8 * kThreads) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + u * kThreads;
                const int r = e / q, c4 = e - r * q;
                v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (e < total && r < rows)
                    v[u] = *reinterpret_cast<const float4*>(src + r * src_stride + 4 * c4);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + u * kThreads;
                if (e < total) {
                    const int r = e / q, c4 = e - r * q;
                    float2* d = reinterpret_cast<float2*>(dst + r * dst_stride + 4 * c4);
                    d[0] = make_float2(v[u].x, v[u].y);
                    d[1] = make_float2(v[u].z, v[u].w);
                }
            }
        }
    } else {
        for (int e = t; e < pad_rows * pad_width; e += kThreads) {
            const int r = e / pad_width, c = e - r * pad_width;
            dst[r * dst_stride + c] = (r < rows && c < width) ? src[r * src_stride + c] : 0.f;
        }
    }
}

// dst[c] = src[c] widened to double for c < valid, 0 beyond (src is read only
// below `valid`).  Float4 loads when the whole span is valid and aligned.
template <int COUNT>
__device__ __forceinline__ void load_span_f64(double (&dst)[COUNT], const float* src, int valid) {
    const bool vec = valid >= COUNT && (reinterpret_cast<uintptr_t>(src) & 15) == 0;
    if (vec) {
#pragma unroll
        for (int m = 0; m < COUNT / 4; ++m) {
            const float4 v = reinterpret_cast<const float4*>(src)[m];
            dst[4 * m] = v.x;
            dst[4 * m + 1] = v.y;
            dst[4 * m + 2] = v.z;
            dst[4 * m + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int c = 0; c < COUNT; ++c) dst[c] = c < valid ? (double)src[c] : 0.0;
    }
}

// The chain's weights: w[j][m] = W_rec[o][64hf + 4j + m] for the forward, or
// (transposed) W_rec[64hf + 4j + m][o] for the backward's W_rec^T; zero outside
// the H x H matrix.  The forward's fast path (H % 4 == 0, W_rec 16-byte aligned)
// is split into fetch (16 float4 loads of the unit's row, from in-range
// addresses, issued together) and widen (masked conversion to double), so that
// the loads can go out early and the widening come later.
__device__ __forceinline__ bool chain_weights_vec(const float* w_rec, int H) {
    return (H & 3) == 0 && (reinterpret_cast<uintptr_t>(w_rec) & 15) == 0;
}
__device__ __forceinline__ void chain_weights_fetch(f32x4 (&raw)[16], const float* __restrict__ w_rec, int H,
                                                    const ChainLane& cl) {
    const float* row = w_rec + (long long)min(cl.o, H - 1) * H;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        raw[j] = *reinterpret_cast<const f32x4*>(row + min(64 * cl.hf + 4 * j, H - 4));
}
__device__ __forceinline__ void chain_weights_widen(double (&w)[16][4], const f32x4 (&raw)[16], int H,
                                                    const ChainLane& cl) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) w[j][m] = cl.o < H && 64 * cl.hf + 4 * j + m < H ? (double)raw[j][m] : 0.0;
}
// The backward's W_rec^T slice in the same two parts: raw[j][m] =
// W_rec[64hf + 4j + m][o] from clamped (in-range) addresses, 64 loads that
// are coalesced across the 16 lanes of a row (consecutive units), then the
// masked widening.  At H = 128 (every index in range) a separate path takes
// constant offsets from one base address and no masks: the general path
// spends four address operations per load and three per widening.
__device__ __forceinline__ void chain_weights_t_fetch(float (&raw)[16][4], const float* __restrict__ w_rec, int H,
                                                      const ChainLane& cl) {
    const long long o = min(cl.o, H - 1);
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) raw[j][m] = w_rec[(long long)min(64 * cl.hf + 4 * j + m, H - 1) * H + o];
}
__device__ __forceinline__ void chain_weights_t_widen(double (&w)[16][4], const float (&raw)[16][4], int H,
                                                      const ChainLane& cl) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) w[j][m] = cl.o < H && 64 * cl.hf + 4 * j + m < H ? (double)raw[j][m] : 0.0;
}
__device__ __forceinline__ void load_chain_weights(double (&w)[16][4], const float* __restrict__ w_rec, int H,
                                                   const ChainLane& cl, bool transposed) {
    if (transposed) {
        float raw[16][4];
        if (H == kSmall) {
            const float* p = w_rec + 64 * cl.hf * kSmall + cl.o;
#pragma unroll
            for (int j = 0; j < 16; ++j)
#pragma unroll
                for (int m = 0; m < 4; ++m) raw[j][m] = p[(4 * j + m) * kSmall];
#pragma unroll
            for (int j = 0; j < 16; ++j)
#pragma unroll
                for (int m = 0; m < 4; ++m) w[j][m] = raw[j][m];
            return;
        }
        chain_weights_t_fetch(raw, w_rec, H, cl);
        chain_weights_t_widen(w, raw, H, cl);
        return;
    }
    if (chain_weights_vec(w_rec, H)) {
        f32x4 raw[16];
        chain_weights_fetch(raw, w_rec, H, cl);
        chain_weights_widen(w, raw, H, cl);
        return;
    }
    const long long o = min(cl.o, H - 1);
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int col = 64 * cl.hf + 4 * j + m;
            w[j][m] = cl.o < H && col < H ? (double)w_rec[o * H + min(col, H - 1)] : 0.0;
        }
}

__global__ __launch_bounds__(kThreads) void cfc_fwd_small_kernel(
    const float* __restrict__ w_in, const float* __restrict__ w_rec,
    const float* __restrict__ bias, const float* __restrict__ w_tau,
    const float* __restrict__ x, const float* __restrict__ h0, double dt, int K, int n_in,
    int H, float* __restrict__ h_seq, int cell) {
    constexpr int HP = kSmall, NP = kSmall, KW = kSmallFwdKW, XS = kSmallXS;
    extern __shared__ __align__(16) unsigned char smem[];
    double* U = reinterpret_cast<double*>(smem);  // [KW][HP]
    double* hb = U + KW * HP;                     // [2][HP]
    int* nonfinite = reinterpret_cast<int*>(hb + 2 * HP);  // the row's flag (16 bytes reserved)
    float* xs = reinterpret_cast<float*>(hb + 2 * HP + 2);  // [KW][XS]

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const long long b = blockIdx.x;
    const ChainLane cl = chain_lane(wave, lane);
    const int o = cl.o;
    const bool gate_lane = cl.gate;
    if (t == 0) *nonfinite = 0;  // read only after the first window's barriers

    // Weight operand of the input projection, kept in registers.  The
    // contraction index of chunk jc in k-slot s = lane/16 is j = 32*s + jc, so a
    // lane's operands are one contiguous span of a W_in row:
    // wb[q][jc] = W_in[(2*wave + q)*16 + lane%16][32*(lane/16) + jc]
    const int slot = lane >> 4;
    double wb[2][NP / 4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = (2 * wave + q) * 16 + (lane & 15);
        const int valid = row < H ? min(max(n_in - 32 * slot, 0), NP / 4) : 0;
        load_span_f64<NP / 4>(wb[q], w_in + (long long)min(row, H - 1) * n_in + min(32 * slot, n_in - 1), valid);
    }
    // W_rec slice for the recurrence
    double wr[16][4];
    load_chain_weights(wr, w_rec, H, cl, false);
    for (int u = t; u < HP; u += kThreads) hb[u] = u < H ? (double)h0[b * H + u] : 0.0;
    const UnitGate ug = unit_gate(cell, o < H ? (double)w_tau[o] : 0.0, dt, o < H);
    double hprev = o < H ? (double)h0[b * H + o] : 0.0;
    const double bias_q0 = (2 * wave) * 16 + (lane & 15) < H ? (double)bias[(2 * wave) * 16 + (lane & 15)] : 0.0;
    const double bias_q1 = (2 * wave + 1) * 16 + (lane & 15) < H ? (double)bias[(2 * wave + 1) * 16 + (lane & 15)] : 0.0;
    // the flag is sticky: once a window has a non-finite input, later windows
    // carry the NaN in their state
    bool bad = any_not_finite(wr) || any_not_finite(ug) || not_finite(hprev);

    int cur = 0;
    for (int k0 = 0; k0 < K; k0 += KW) {
        const int kw = min(KW, K - k0);
        __syncthreads();  // the previous window is done with xs and U
        stage_rows(xs, XS, x + (b * K + k0) * (long long)n_in, n_in, kw, n_in, KW, NP, t);
        __syncthreads();
        // ---- input projection of the window on the matrix cores
        {
            dbl4 acc[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[kb][q] = dbl4{0.0, 0.0, 0.0, 0.0};
            const float* xa = xs + (lane & 15) * XS + 32 * slot;
#pragma unroll
            for (int jc = 0; jc < NP / 4; ++jc) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const double a = (double)xa[kb * 16 * XS + jc];
                    acc[kb][0] = mfma_f64(a, wb[0][jc], acc[kb][0]);
                    acc[kb][1] = mfma_f64(a, wb[1][jc], acc[kb][1]);
                }
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    double* urow = U + (kb * 16 + (lane >> 4) + 4 * v) * HP + (2 * wave) * 16 + (lane & 15);
                    // stored as a quarter: it seeds both accumulators of both
                    // lanes of the unit's pair in the chain product
                    const double u0 = acc[kb][0][v] + bias_q0, u1 = acc[kb][1][v] + bias_q1;
                    urow[0] = 0.25 * u0;
                    urow[16] = 0.25 * u1;
                    bad |= not_finite(u0) || not_finite(u1);
                }
        }
        const GateLane gl = gate_lane_consts(gate_lane, ug);
        if (bad) *nonfinite = 1;
        __syncthreads();
        // ---- serial recurrence through the window
        auto chain = [&](auto exact) {
            constexpr bool EXACT = decltype(exact)::value;
            const double zl = gl.zmul * kLog2e;
            for (int kk = 0; kk < kw; ++kk) {
                lds_and_scalar_drained();
                const double u4 = U[kk * HP + o];
                double hs[4];
                chain_read(hs, hb + cur * HP, cl);
                const double a = chain_total(chain_product(wr, hs, u4));
                double g, c;
                cell_gates_t<EXACT>(a, gl, zl, g, c);
                const double hn = fma(g, hprev - c, c);  // g*h + (1-g)*c
                hprev = hn;
                // both lanes of the unit's pair hold the same bits (the last
                // reduce stage adds the same two values, and g, c are exchanged),
                // so both store: no branch in the loop
                hb[(cur ^ 1) * HP + o] = hn;
                if (o < H) h_seq[(b * K + k0 + kk) * (long long)H + o] = (float)hn;
                cur ^= 1;
                __syncthreads();
            }
        };
        if (*nonfinite)
            chain(std::true_type{});
        else
            chain(std::false_type{});
    }
}

__device__ __forceinline__ void store_grad_f(float* p, double v, int accumulate) {
    *p = accumulate ? (float)v + *p : (float)v;
}

// Second half of a row's backward pass, shared by cfc_bwd_small_kernel and
// cfc_fb_small_kernel.  On entry (after a barrier): AD[k][*] holds a_k for
// k < K and 0 beyond, zs[k] holds [x_k | h_k-1] (rows >= K zero), ug is the
// gate of this lane's unit o, and delta is h_K - y of unit o (computed from the
// float32 h_K).  Seeds the row's loss, runs the reverse
// chain (AD[k] becomes dL/da_k), forms G = DA^T [X | H_prev] on the matrix
// cores and writes the row [dW_in | dW_rec | db | dw_tau].  Optionally also
// the input gradients of the row: gh0_row [H] = dL/dh_0 (the chain runs its
// W_rec^T step once more, at k = 0) and gx_row [K][n_in] = DA W_in (a third
// product on the matrix cores).  red[4] holds the row's non-finite flag as an
// int (zeroed before an earlier barrier); `bad` is this thread's own test of
// what the pre-activations in AD were formed from.
__device__ __forceinline__ void small_reverse_and_grads(
    const float* __restrict__ w_in, const float* __restrict__ w_rec, int K, int n_in, int H,
    double delta, double* AD, const UnitGate& ug, double* red, const float* zs,
    float* gst, float* __restrict__ row, float* __restrict__ loss_b, float* __restrict__ gx_row,
    float* __restrict__ gh0_row, int accumulate, int lane, int wave, const ChainLane& cl, bool bad) {
    constexpr int HP = kSmall, NP = kSmall, ZW = kSmallZW, ZS = kSmallZS, AS = kSmallAS;
    constexpr int KP = kSmallBwdMaxK;
    int* nonfinite = reinterpret_cast<int*>(red + 4);
    const int o = cl.o;
    const bool gate_lane = cl.gate;
    // ---- W_rec^T slice into registers.  Its values need no finiteness test
    // here: both callers' pre-activations contract all of W_rec, and a
    // non-finite weight makes them non-finite (inf times 0 is NaN), which the
    // callers have flagged.
    double wt[16][4];
    load_chain_weights(wt, w_rec, H, cl, true);
    if (bad || any_not_finite(ug)) *nonfinite = 1;

    // ---- loss seed
    {
        const double l = wave_sum_f64(gate_lane ? 0.0 : 0.5 * delta * delta);
        if (lane == 0) red[wave] = l;
    }
    const GateLane gl = gate_lane_consts(gate_lane, ug);
    __syncthreads();
    if (wave == 0 && lane == 0 && loss_b) *loss_b = (float)(((red[0] + red[1]) + red[2]) + red[3]);

    // ---- serial reverse chain.  Per step only delta carries a dependency:
    // dz = delta P, dL/da = delta Q, the dw_tau term = delta R, with g, P, Q,
    // R functions of a_k and h_k alone; they are computed one step ahead,
    // after the barrier, while the step's LDS reads and products are in
    // flight.  a_k-1 is still in AD when they are read (it is overwritten by
    // dL/da_k-1 one step later, by the same lane pair).
    double gb = 0.0, gwt = 0.0;
    auto reverse_chain = [&](auto exact) {
        constexpr bool EXACT = decltype(exact)::value;
        const double zl = gl.zmul * kLog2e;
        // g4 = g / 4: delta g seeds both accumulators of both lanes of the
        // unit's pair in the chain product as a quarter each
        auto step_consts = [&](int k, double& g4, double& Q, double& R) {
            const double a = AD[k * AS + o];
            const double hk = (double)zs[k * ZS + NP + o];
            double g, c;
            cell_gates_t<EXACT>(a, gl, zl, g, c);
            const double P = (hk - c) * g * fma(-ug.vmul, g, 1.0);
            Q = (1.0 - g) * (1.0 - c * c) - P * ug.rho;
            R = P * fma(-a, ug.alpha, ug.beta);
            g4 = 0.25 * g;
        };
        double g4, Q, R;
        step_consts(K - 1, g4, Q, R);
        for (int k = K - 1; k >= 0; --k) {
            const double da = delta * Q;
            gb += da;
            gwt += delta * R;
            if (!gate_lane) AD[k * AS + o] = da;
            __syncthreads();
            if (k == 0 && !gh0_row) break;
            double ds[4];
            chain_read(ds, AD + k * AS, cl);
            // next step's constants (unused after k = 0), in the same block as
            // the products so that their latency overlaps them
            double g4n, Qn, Rn;
            step_consts(k > 0 ? k - 1 : 0, g4n, Qn, Rn);
            delta = chain_total(chain_product(wt, ds, delta * g4));  // delta g + W_rec^T dL/da_k
            g4 = g4n;
            Q = Qn;
            R = Rn;
        }
    };
    if (*nonfinite)
        reverse_chain(std::true_type{});
    else
        reverse_chain(std::false_type{});
    if (gh0_row && !gate_lane && o < H) gh0_row[o] = (float)delta;  // dL/dh_0

    // ---- weight gradients on the matrix cores: G = DA^T [X | H_prev]
    float* rrec = row + (long long)H * n_in;
    {
        const int ib0 = 2 * wave;
        constexpr int KC = KP / 4;
        const double* ada = AD + (lane >> 4) * AS + ib0 * 16 + (lane & 15);
        const float* zb = zs + (lane >> 4) * ZS + (lane & 15);
        // Exactly 128 x 128 with 16-byte-aligned rows (either mode): no
        // masking, and each group's tiles are stored while the next group's
        // products run (the groups' stores otherwise wait for their products).
        // The float4 stores are non-temporal: the scratch is written once
        // and read next by the reducer; measured on MI355X at B = 256, the
        // fused kernel took 79.8 against 81.0 us and the reduce after it
        // 10.5 against 11.6 us, against ordinary stores.
        const bool interleave = n_in == NP && H == HP && (reinterpret_cast<uintptr_t>(row) & 15) == 0;
        if (interleave) {
            const int c4 = 4 * (lane & 15);
            // the previous group's tiles (float32, MFMA layout) and one step
            // of their store: kc 0..3 / 8..11 write tile q's columns jj = kc % 4
            // into the wave's LDS buffer, kc 4..7 / 12..15 read back row
            // block m = kc % 4 transposed and store it (float4, 256 bytes per
            // 16 lanes).  Accumulate mode loads the old values of row block m
            // four chunks ahead (at kc m / 8 + m) and adds the float32 tile to
            // them in float32, as a float32 += into the scratch would.
            // one instance of the loop per mode, so neither carries a branch
            auto run = [&](auto acc_mode) {
                constexpr bool ACC = decltype(acc_mode)::value;
                float pend[2][4][4];
                float4 old4[4];
                auto dst_of = [&](int jgp, int q, int m) -> float* {
                    const int i = (ib0 + q) * 16 + (lane >> 4) + 4 * m;
                    const int jc0 = jgp * 64 + c4;
                    return jc0 < NP ? row + (long long)i * NP + jc0 : rrec + (long long)i * HP + (jc0 - NP);
                };
                auto store_step = [&](int jgp, int kc) {
                    const int q = kc >> 3, st = kc & 7;
                    if (st < 4) {
                        if constexpr (ACC) old4[st] = *reinterpret_cast<const float4*>(dst_of(jgp, q, st));
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            gst[((lane >> 4) + 4 * v) * kSmallGS + st * 16 + (lane & 15)] = pend[q][st][v];
                    } else {
                        const int m = st - 4, r = (lane >> 4) + 4 * m;
                        float4 val = *reinterpret_cast<const float4*>(gst + r * kSmallGS + c4);
                        if constexpr (ACC) {
                            const float4 o = old4[m];
                            val = make_float4(val.x + o.x, val.y + o.y, val.z + o.z, val.w + o.w);
                        }
                        __builtin_nontemporal_store(f32x4{val.x, val.y, val.z, val.w},
                                                    reinterpret_cast<f32x4*>(dst_of(jgp, q, m)));
                    }
                };
                for (int jg = 0; jg < ZW / 64; ++jg) {
                    dbl4 acc[2][4];
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) acc[q][jj] = dbl4{0.0, 0.0, 0.0, 0.0};
                    double a0 = ada[0], a1 = ada[16];
                    double bz[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) bz[jj] = (double)zb[(jg * 4 + jj) * 16];
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        const int kn = kc + 1 < KC ? kc + 1 : kc;
                        const double na0 = ada[4 * kn * AS], na1 = ada[4 * kn * AS + 16];
                        double nbz[4];
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) nbz[jj] = (double)zb[4 * kn * ZS + (jg * 4 + jj) * 16];
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            acc[0][jj] = mfma_f64(a0, bz[jj], acc[0][jj]);
                            acc[1][jj] = mfma_f64(a1, bz[jj], acc[1][jj]);
                        }
                        if (jg > 0) store_step(jg - 1, kc);
                        a0 = na0;
                        a1 = na1;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) bz[jj] = nbz[jj];
                    }
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                            for (int v = 0; v < 4; ++v) pend[q][jj][v] = (float)acc[q][jj][v];
                }
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) store_step(ZW / 64 - 1, kc);
            };
            if (accumulate)
                run(std::integral_constant<bool, true>{});
            else
                run(std::integral_constant<bool, false>{});
        }
        for (int jg = 0; jg < (interleave ? 0 : ZW / 64); ++jg) {
            dbl4 acc[2][4];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[q][jj] = dbl4{0.0, 0.0, 0.0, 0.0};
            // operands of chunk kc: rows 4kc + lane/16
            double a0 = ada[0], a1 = ada[16];
            double bz[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) bz[jj] = (double)zb[(jg * 4 + jj) * 16];
            for (int kc = 0; kc < KC; ++kc) {
                const int kn = kc + 1 < KC ? kc + 1 : kc;
                const double na0 = ada[4 * kn * AS], na1 = ada[4 * kn * AS + 16];
                double nbz[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) nbz[jj] = (double)zb[4 * kn * ZS + (jg * 4 + jj) * 16];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    acc[0][jj] = mfma_f64(a0, bz[jj], acc[0][jj]);
                    acc[1][jj] = mfma_f64(a1, bz[jj], acc[1][jj]);
                }
                a0 = na0;
                a1 = na1;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) bz[jj] = nbz[jj];
            }
            if (accumulate) {
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int jcol = (jg * 4 + jj) * 16 + (lane & 15);
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int i = (ib0 + q) * 16 + (lane >> 4) + 4 * v;
                            if (i >= H) continue;
                            if (jcol < NP) {
                                if (jcol < n_in) store_grad_f(row + (long long)i * n_in + jcol, acc[q][jj][v], 1);
                            } else if (jcol - NP < H) {
                                store_grad_f(rrec + (long long)i * H + (jcol - NP), acc[q][jj][v], 1);
                            }
                        }
                    }
            } else {
                // Through the wave's LDS buffer: each 16 x 64 block of G is
                // transposed from the MFMA layout into rows, then stored as
                // row-contiguous float4 (256 bytes per 16 lanes).
                const int c4 = 4 * (lane & 15);       // first of this lane's 4 columns
                const int jc0 = jg * 64 + c4;         // its column of [X | H_prev]
                const bool in_part = jc0 < NP;
                const int col = in_part ? jc0 : jc0 - NP;
                const int width = in_part ? n_in : H;
                float* base = in_part ? row : rrec;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            gst[((lane >> 4) + 4 * v) * kSmallGS + jj * 16 + (lane & 15)] = (float)acc[q][jj][v];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int r = (lane >> 4) + 4 * m;
                        const float4 val = *reinterpret_cast<const float4*>(gst + r * kSmallGS + c4);
                        const int i = (ib0 + q) * 16 + r;
                        if (i < H) {
                            float* dst = base + (long long)i * width + col;
                            if (col + 4 <= width && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                                *reinterpret_cast<float4*>(dst) = val;
                            } else {
                                if (col < width) dst[0] = val.x;
                                if (col + 1 < width) dst[1] = val.y;
                                if (col + 2 < width) dst[2] = val.z;
                                if (col + 3 < width) dst[3] = val.w;
                            }
                        }
                    }
                }
            }
        }
    }
    if (!gate_lane && o < H) {
        store_grad_f(rrec + (long long)H * H + o, gb, accumulate);
        store_grad_f(rrec + (long long)H * H + H + o, gwt, accumulate);
    }

    // ---- input gradient GX = DA W_in on the matrix cores: wave w owns the
    // column tiles jt = 2w, 2w+1 of n_in for all four 16-step tiles; chunk c
    // contracts i = 4c + lane/16 (A = DA[16kt + lane%16][i] from LDS,
    // B = W_in[i][16jt + lane%16] from L2)
    if (gx_row) {
        const int m = lane & 15, q = lane >> 4;
        // the wave's whole W_in operand (both column tiles, 64 floats per
        // lane) is loaded first, so its latency is exposed once
        float wv[2][HP / 4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = (2 * wave + jj) * 16 + m;
#pragma unroll
            for (int c = 0; c < HP / 4; ++c) {
                const int i = 4 * c + q;
                wv[jj][c] = (i < H && j < n_in) ? w_in[(long long)i * n_in + j] : 0.f;
            }
        }
#pragma unroll 1
        for (int jj = 0; jj < 2; ++jj) {
            const int j = (2 * wave + jj) * 16 + m;
            dbl4 acc[KP / 16];
#pragma unroll
            for (int kt = 0; kt < KP / 16; ++kt) acc[kt] = dbl4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int c = 0; c < HP / 4; ++c) {
                const int i = 4 * c + q;
                const double w = (double)(jj == 0 ? wv[0][c] : wv[1][c]);
#pragma unroll
                for (int kt = 0; kt < KP / 16; ++kt) acc[kt] = mfma_f64(AD[(kt * 16 + m) * AS + i], w, acc[kt]);
            }
            if (j < n_in) {
#pragma unroll
                for (int kt = 0; kt < KP / 16; ++kt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int k = kt * 16 + q + 4 * v;
                        if (k < K) gx_row[(long long)k * n_in + j] = (float)acc[kt][v];
                    }
            }
        }
    }
}

// WHOLE: a 64-step window, n_in = n_hid = 128, and x, h0, h_seq, W_in, W_rec
// 16-byte aligned (the host checks): the staging then runs unconditionally
// and fetches the recomputation's weights while [x | h_prev] is staged (x and
// h first, then the per-unit inputs, then the weights: vmcnt retires in
// order), widening them after the barrier.  A separate instance, so that no
// path joins the generic one.
template <bool WHOLE>
__global__ __launch_bounds__(kThreads) void cfc_bwd_small_kernel(
    const float* __restrict__ w_in, const float* __restrict__ w_rec,
    const float* __restrict__ bias, const float* __restrict__ w_tau,
    const float* __restrict__ x, const float* __restrict__ h0, const float* __restrict__ h_seq,
    const float* __restrict__ y, double dt, BwdWindow win, int n_in, int H, float* __restrict__ scratch,
    float* __restrict__ loss, float* __restrict__ grad_x, int accumulate, int cell) {
    constexpr int HP = kSmall, NP = kSmall, ZW = kSmallZW, ZS = kSmallZS;
    const int K = win.Kw;  // steps of this launch; indices below are relative to win.k0
    const long long Kf = win.K, k0 = win.k0;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KP = kSmallBwdMaxK;
    constexpr int AS = kSmallAS;
    double* AD = reinterpret_cast<double*>(smem);  // [KP][AS]: a, then dL/da
    double* red = AD + KP * AS;                    // [8]
    float* zs = reinterpret_cast<float*>(red + 8);  // [KP][ZS] = [x_k | h_k]

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float* gst = zs + KP * ZS + wave * 16 * kSmallGS;  // this wave's [16][kSmallGS] tile buffer
    const long long b = blockIdx.x;
    const long long N = (long long)H * (n_in + H + 2);
    const ChainLane cl = chain_lane(wave, lane);
    const int o = cl.o;
    if (t == 0) reinterpret_cast<int*>(red + 4)[0] = 0;  // the row's non-finite flag

    // Weight operand of the recomputation, in registers.  Chunk jc of k-slot
    // s = lane/16 contracts index j = 64*s + jc of [x | h_prev], so a lane holds
    // one contiguous 64-wide span of a row of W_in (s = 0, 1) or W_rec (s = 2, 3):
    // wb[q][jc] = [W_in | W_rec][(2*wave + q)*16 + lane%16][64*s + jc]
    const int slot = lane >> 4;
    double wb[2][ZW / 4];
    auto load_weights = [&]() {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = (2 * wave + q) * 16 + (lane & 15);
            const int rowc = min(row, H - 1);
            const bool in_part = slot < 2;
            const int c0 = in_part ? 64 * slot : 64 * (slot - 2);
            const int width = in_part ? n_in : H;
            const int valid = row < H ? min(max(width - c0, 0), ZW / 4) : 0;
            const float* src = in_part ? w_in + (long long)rowc * n_in + min(c0, n_in - 1)
                                       : w_rec + (long long)rowc * H + min(c0, H - 1);
            load_span_f64<ZW / 4>(wb[q], src, valid);
        }
    };
    float wtau_o, bias0, bias1;
    const int bcol0 = (2 * wave) * 16 + (lane & 15), bcol1 = bcol0 + 16;
    f32x4 wpre[2][ZW / 16];
    if constexpr (WHOLE) {
        // ---- stage [x_k | h_k]: KP rows of ZW / 4 float4, x in the first
        // NP / 4 of them (8 per thread), h in the rest (8 per thread; row 0 is
        // h_k0-1, from h0 when the window starts the sequence)
        static_assert(KP * (NP / 4) == 8 * kThreads && KP * (HP / 4) == 8 * kThreads, "one pass per half");
        const f32x4* xb = reinterpret_cast<const f32x4*>(x + (b * Kf + k0) * NP);
        const float* h_first = k0 == 0 ? h0 + b * HP : h_seq + (b * Kf + k0 - 1) * HP;
        const float* h_rest = h_seq + (b * Kf + k0) * HP;  // row r >= 1 is h_rest[r - 1]
        f32x4 xv[8], hv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = t + u * kThreads;
            xv[u] = xb[e];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = t + u * kThreads, r = e / (HP / 4), c4 = e % (HP / 4);
            const float* src = r == 0 ? h_first : h_rest + (r - 1) * HP;
            hv[u] = reinterpret_cast<const f32x4*>(src)[c4];
        }
        wtau_o = w_tau[o];
        bias0 = bias[bcol0];
        bias1 = bias[bcol1];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = (2 * wave + q) * 16 + (lane & 15);
            const float* src = slot < 2 ? w_in + row * NP + 64 * slot : w_rec + row * HP + 64 * (slot - 2);
#pragma unroll
            for (int m = 0; m < ZW / 16; ++m) wpre[q][m] = reinterpret_cast<const f32x4*>(src)[m];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = t + u * kThreads, r = e / (NP / 4), c4 = e % (NP / 4);
            float2* dx = reinterpret_cast<float2*>(zs + r * ZS + 4 * c4);
            dx[0] = make_float2(xv[u][0], xv[u][1]);
            dx[1] = make_float2(xv[u][2], xv[u][3]);
            float2* dh = reinterpret_cast<float2*>(zs + r * ZS + NP + 4 * c4);
            dh[0] = make_float2(hv[u][0], hv[u][1]);
            dh[1] = make_float2(hv[u][2], hv[u][3]);
        }
    } else {
        (void)wpre;
        load_weights();
        // ---- stage [x_k | h_k] for every step of the window (h_0 = h0, h_k = h_seq[k-1])
        stage_rows(zs, ZS, x + (b * Kf + k0) * n_in, n_in, K, n_in, KP, NP, t);
        stage_rows(zs + NP, ZS, k0 == 0 ? h0 + b * H : h_seq + (b * Kf + k0 - 1) * H, H, 1, H, 1, HP, t);
        if (K > 1) stage_rows(zs + ZS + NP, ZS, h_seq + (b * Kf + k0) * H, H, K - 1, H, KP - 1, HP, t);
        else stage_rows(zs + ZS + NP, ZS, h_seq, H, 0, H, KP - 1, HP, t);
        wtau_o = o < H ? w_tau[o] : 0.f;
        bias0 = bcol0 < H ? bias[bcol0] : 0.f;
        bias1 = bcol1 < H ? bias[bcol1] : 0.f;
    }
    const UnitGate ug = unit_gate(cell, (double)wtau_o, dt, WHOLE || o < H);  // o < 128 = H in WHOLE
    const double bias_q0 = bias0, bias_q1 = bias1;
    __syncthreads();
    if constexpr (WHOLE) {
        // the empty asm takes the loaded registers here, after the barrier,
        // so the wait for them and their widening are not hoisted above it
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int m = 0; m < ZW / 16; ++m) {
                asm volatile("" : "+v"(wpre[q][m]));
#pragma unroll
                for (int e = 0; e < 4; ++e) wb[q][4 * m + e] = wpre[q][m][e];
            }
    }

    // ---- recompute every step's pre-activation on the matrix cores
    bool bad = false;
    {
        dbl4 acc[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[kb][q] = dbl4{0.0, 0.0, 0.0, 0.0};
        const float* za = zs + (lane & 15) * ZS + 64 * slot;
#pragma unroll
        for (int jc = 0; jc < ZW / 4; ++jc) {
#pragma unroll
            for (int kb = 0; kb < KP / 16; ++kb) {
                const double a = (double)za[kb * 16 * ZS + jc];
                acc[kb][0] = mfma_f64(a, wb[0][jc], acc[kb][0]);
                acc[kb][1] = mfma_f64(a, wb[1][jc], acc[kb][1]);
            }
        }
#pragma unroll
        for (int kb = 0; kb < KP / 16; ++kb) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int kk = kb * 16 + (lane >> 4) + 4 * v;
                double* arow = AD + kk * AS + (2 * wave) * 16 + (lane & 15);
                const double a0 = kk < K ? acc[kb][0][v] + bias_q0 : 0.0;
                const double a1 = kk < K ? acc[kb][1][v] + bias_q1 : 0.0;
                arow[0] = a0;
                arow[16] = a1;
                bad |= not_finite(a0) || not_finite(a1);
            }
        }
    }

    const double delta = o >= H ? 0.0
                         : win.delta_in ? (double)win.delta_in[b * H + o]
                                        : (double)h_seq[(b * Kf + Kf - 1) * H + o] - (double)y[b * H + o];
    small_reverse_and_grads(w_in, w_rec, K, n_in, H, delta, AD, ug, red, zs, gst, scratch + b * N,
                            loss && !win.delta_in ? loss + b : nullptr,
                            grad_x ? grad_x + (b * Kf + k0) * n_in : nullptr,
                            win.delta_out ? win.delta_out + b * H : nullptr, accumulate, lane, wave, cl, bad);
}

// Forward and backward of one row in one workgroup (n_in, n_hid <= 128,
// K <= 64).  The forward's pre-activations a_k stay in LDS (in float64) for the
// reverse chain and [x_k | h_k-1] is staged once for both directions, so
// nothing is recomputed and nothing is read back from h_seq.
__host__ __device__ constexpr size_t small_fb_lds_bytes() {
    return small_bwd_lds_bytes() + (size_t)8 * 2 * kSmall;
}

// WHOLE: K = 64, n_in = n_hid = 128, W_in and x 16-byte aligned (the host
// checks); the staging then runs with no guards and fetches the projection's
// weights while x is staged.  A separate instance, so that no code path joins
// the generic one (where the wait for the staging's loads would be merged
// conservatively into a wait for all of them).
template <bool WHOLE>
__global__ __launch_bounds__(kThreads) void cfc_fb_small_kernel(
    const float* __restrict__ w_in, const float* __restrict__ w_rec,
    const float* __restrict__ bias, const float* __restrict__ w_tau,
    const float* __restrict__ x, const float* __restrict__ h0, const float* __restrict__ y, double dt,
    int K, int n_in, int H, float* __restrict__ h_seq, float* __restrict__ scratch,
    float* __restrict__ loss, float* __restrict__ grad_x, float* __restrict__ grad_h0, int accumulate,
    int cell) {
    constexpr int HP = kSmall, NP = kSmall, ZS = kSmallZS, KP = kSmallBwdMaxK;
    // the shared reverse pass gets the sizes as passed; the instance's own
    // phases take them as constants
    const int K_arg = K, n_in_arg = n_in, H_arg = H;
    if constexpr (WHOLE) {
        K = KP;
        n_in = NP;
        H = HP;
    }
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int AS = kSmallAS;
    double* AD = reinterpret_cast<double*>(smem);  // [KP][AS]: W_in x_k + b, then a_k, then dL/da_k
    double* red = AD + KP * AS;                    // [8]
    double* hb = red + 8;                          // [2][HP] h_k exchange
    float* zs = reinterpret_cast<float*>(hb + 2 * HP);  // [KP][ZS] = [x_k | h_k-1]

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float* gst = zs + KP * ZS + wave * 16 * kSmallGS;
    const long long b = blockIdx.x;
    const long long N = (long long)H * (n_in + H + 2);
    const ChainLane cl = chain_lane(wave, lane);
    const int o = cl.o;
    const bool gate_lane = cl.gate;
    const int slot = lane >> 4;
    int* nonfinite = reinterpret_cast<int*>(red + 4);
    if (t == 0) *nonfinite = 0;

    // ---- stage x (rows >= K zero), h0 as row 0 of the h_prev half (rows >= K
    // zero; rows 1..K-1 are written by the chain), per-unit constants
    // In the WHOLE instance the projection's weight operand (below) is fetched
    // while x is staged: x's loads go first, then the small per-unit ones,
    // then W_in's, then x's LDS writes, which wait for x's loads only.
    const float* xb = x + b * K * (long long)n_in;
    f32x4 wpre[2][NP / 16];
    // the per-unit inputs, as floats: w_tau, h_0 and y of unit o, the bias
    // of the projection's two output columns
    float wtau_o, h0_o, y_o, bias0, bias1;
    f32x4 wr_raw[16];    // WHOLE: the forward chain's W_rec slice, fetched under the projection
    const int bcol0 = (2 * wave) * 16 + (lane & 15), bcol1 = bcol0 + 16;
    if constexpr (WHOLE) {
        // every load is unconditional (all indices are in range here), and
        // all go out before W_in's 16 float4 (vmcnt retires in order)
        static_assert(KP * (NP / 4) == 8 * kThreads, "one pass of 8 float4 per thread");
        f32x4 xv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) xv[u] = reinterpret_cast<const f32x4*>(xb)[t + u * kThreads];
        const float h0_t = h0[b * H + (t & (HP - 1))];
        wtau_o = w_tau[o];
        h0_o = h0[b * H + o];
        bias0 = bias[bcol0];
        bias1 = bias[bcol1];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const f32x4* src = reinterpret_cast<const f32x4*>(w_in + ((2 * wave + q) * 16 + (lane & 15)) * NP + 32 * slot);
#pragma unroll
            for (int m = 0; m < NP / 16; ++m) wpre[q][m] = src[m];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = t + u * kThreads, r = e / (NP / 4), c4 = e % (NP / 4);
            float2* d = reinterpret_cast<float2*>(zs + r * ZS + 4 * c4);
            d[0] = make_float2(xv[u][0], xv[u][1]);
            d[1] = make_float2(xv[u][2], xv[u][3]);
        }
        // h_0 into row 0's h_prev half and the h exchange (threads t and
        // t + 128 write the same value)
        zs[NP + (t & (HP - 1))] = h0_t;
        hb[t & (HP - 1)] = (double)h0_t;
    } else {
        (void)wpre;
        stage_rows(zs, ZS, xb, n_in, K, n_in, KP, NP, t);
        stage_rows(zs + NP, ZS, h0 + b * H, H, 1, H, 1, HP, t);
        stage_rows(zs + K * ZS + NP, ZS, h0, H, 0, H, KP - K, HP, t);
        for (int u = t; u < HP; u += kThreads) hb[u] = u < H ? (double)h0[b * H + u] : 0.0;
        wtau_o = o < H ? w_tau[o] : 0.f;
        h0_o = o < H ? h0[b * H + o] : 0.f;
        y_o = o < H ? y[b * H + o] : 0.f;
        (void)wr_raw;
        bias0 = bcol0 < H ? bias[bcol0] : 0.f;
        bias1 = bcol1 < H ? bias[bcol1] : 0.f;
    }
    const UnitGate ug = unit_gate(cell, (double)wtau_o, dt, WHOLE || o < H);  // o < 128 = H in WHOLE
    const double bias_q0 = bias0, bias_q1 = bias1;
    __syncthreads();

    // ---- input projection of all K steps on the matrix cores: chunk jc of
    // k-slot s contracts j = 32*s + jc, a contiguous span of a W_in row
    bool bad = false;
    {
        double wb[2][NP / 4];
        if constexpr (WHOLE) {
            // the forward chain's weights and the loss target stream in
            // under the products; W_in's float4 are taken one chunk group
            // at a time inside the product loop (below), so that the products
            // start as the first of them arrive
            chain_weights_fetch(wr_raw, w_rec, HP, cl);
            y_o = y[b * H + o];
        } else {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int row = (2 * wave + q) * 16 + (lane & 15);
                const int valid = row < H ? min(max(n_in - 32 * slot, 0), NP / 4) : 0;
                load_span_f64<NP / 4>(wb[q], w_in + (long long)min(row, H - 1) * n_in + min(32 * slot, n_in - 1),
                                      valid);
            }
        }
        dbl4 acc[KP / 16][2];
#pragma unroll
        for (int kb = 0; kb < KP / 16; ++kb)
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[kb][q] = dbl4{0.0, 0.0, 0.0, 0.0};
        const float* xa = zs + (lane & 15) * ZS + 32 * slot;
#pragma unroll
        for (int jc = 0; jc < NP / 4; ++jc) {
            if constexpr (WHOLE) {
                if (jc % 4 == 0) {
                    // the empty asm takes float4 jc / 4 of both rows here, so
                    // the wait for it and its widening are not hoisted
                    const int m = jc / 4;
                    asm volatile("" : "+v"(wpre[0][m]), "+v"(wpre[1][m]));
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) wb[q][4 * m + e] = wpre[q][m][e];
                }
            }
#pragma unroll
            for (int kb = 0; kb < KP / 16; ++kb) {
                const double a = (double)xa[kb * 16 * ZS + jc];
                acc[kb][0] = mfma_f64(a, wb[0][jc], acc[kb][0]);
                acc[kb][1] = mfma_f64(a, wb[1][jc], acc[kb][1]);
            }
        }
#pragma unroll
        for (int kb = 0; kb < KP / 16; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int kk = kb * 16 + (lane >> 4) + 4 * v;
                double* urow = AD + kk * AS + (2 * wave) * 16 + (lane & 15);
                // stored as a quarter: it seeds both accumulators of both lanes
                // of the unit's pair in the forward chain's product
                const double u0 = kk < K ? acc[kb][0][v] + bias_q0 : 0.0;
                const double u1 = kk < K ? acc[kb][1][v] + bias_q1 : 0.0;
                urow[0] = 0.25 * u0;
                urow[16] = 0.25 * u1;
                bad |= not_finite(u0) || not_finite(u1);
            }
    }

    // ---- forward chain (as in cfc_fwd_small_kernel); a_k replaces the
    // projection in AD, h_k goes to h_seq and to the h_prev half of row k+1
    double wr[16][4];
    if constexpr (WHOLE) {
        // as with W_in: the wait and the widening stay here
#pragma unroll
        for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(wr_raw[j]));
        chain_weights_widen(wr, wr_raw, H, cl);
    } else {
        load_chain_weights(wr, w_rec, H, cl, false);
    }
    double hprev = h0_o;
    const GateLane gl = gate_lane_consts(gate_lane, ug);
    if (bad || any_not_finite(wr) || any_not_finite(ug) || not_finite(hprev)) *nonfinite = 1;
    __syncthreads();
    auto forward_chain = [&](auto exact) {
        constexpr bool EXACT = decltype(exact)::value;
        const double zl = gl.zmul * kLog2e;
        int cur = 0;
        for (int k = 0; k < K; ++k) {
            lds_and_scalar_drained();
            const double u4 = AD[k * AS + o];
            double hs[4];
            chain_read(hs, hb + cur * HP, cl);
            const double a = chain_total(chain_product(wr, hs, u4));
            double g, c;
            cell_gates_t<EXACT>(a, gl, zl, g, c);
            const double hn = fma(g, hprev - c, c);
            hprev = hn;
            // both lanes of the pair hold the same bits: both store, no branch.
            // The state the next step reads goes first; the scheduling barrier
            // keeps the other stores' conversions from being hoisted above it.
            hb[(cur ^ 1) * HP + o] = hn;
            __builtin_amdgcn_sched_barrier(0);
            AD[k * AS + o] = a;
            if (k + 1 < K) zs[(k + 1) * ZS + NP + o] = (float)hn;
            if (o < H) h_seq[(b * K + k) * (long long)H + o] = (float)hn;
            cur ^= 1;
            __syncthreads();
        }
    };
    if (*nonfinite)
        forward_chain(std::true_type{});
    else
        forward_chain(std::false_type{});

    // ---- backward from the float32 h_K, as the separate backward sees it
    const double delta = o < H ? (double)(float)hprev - (double)y_o : 0.0;
    small_reverse_and_grads(w_in, w_rec, K_arg, n_in_arg, H_arg, delta, AD, ug, red, zs, gst, scratch + b * N,
                            loss ? loss + b : nullptr, grad_x ? grad_x + b * K * (long long)n_in : nullptr,
                            grad_h0 ? grad_h0 + b * H : nullptr, accumulate, lane, wave, cl, false);
}

// =====================================================================
// Kernels for 128 < max(n_in, n_hid) <= 256 (the large-batch workload).  A
// workgroup owns kLR = 16 batch rows, so each step's contraction
// [W_in | W_rec] (256 x 512) x [x_k ; h_k] (512 x 16 rows) is a dense product
// on the f64 matrix cores, as is the backward's W_rec^T x dL/da; dimensions
// are zero-padded to 256.  Rows stay independent: the 16 rows only share the
// weight operand of each product.
// =====================================================================
constexpr int kLarge = 256;  // padded n_in and n_hid
// The fourth word of a gfx9 buffer descriptor for raw, untyped access
// (32-bit data format, no swizzle): the weight operands of the wide kernels
// are read through buffer descriptors, whose base sits in scalar registers,
// so each load needs only a 32-bit lane offset and a scalar or immediate one.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kLR = 16;      // batch rows per workgroup
constexpr int kLargeBwdMaxK = 20;

// Element (j, r) of a [256][16] LDS array, XOR-swizzled within each row of 16
// so that an MFMA operand read (16 consecutive r) and a staging write (16
// consecutive j) both touch distinct banks.
__device__ __forceinline__ int zidx(int j, int r) { return j * kLR + (r ^ (j & 15)); }

// Unit held at row m of a wave's output tile tb: the four tiles of a wave
// interleave (units 64*wave + 4*m + tb), so the W_rec^T operand of all four
// tiles is one float4 per lane.
__device__ __forceinline__ int lunit(int wave, int tb, int m) { return 64 * wave + 4 * m + tb; }

// Per-thread slice (16 elements) of rows r0..r0+15 of a [rows][width] matrix:
// element m of thread t is (row (t + 256 m) / 256, column (t + 256 m) % 256).
__device__ __forceinline__ void fetch_t(float (&v)[kLR], const float* src, long long stride, long long r0,
                                        long long B, int width, int t) {
#pragma unroll
    for (int m = 0; m < kLR; ++m) {
        const int e = t + kThreads * m;
        const int rr = e >> 8, j = e & 255;
        const long long b = r0 + rr;
        v[m] = (b < B && j < width) ? src[b * stride + j] : 0.f;
    }
}
template <typename T>
__device__ __forceinline__ void store_t(T* dst, const float (&v)[kLR], int t) {
#pragma unroll
    for (int m = 0; m < kLR; ++m) {
        const int e = t + kThreads * m;
        dst[zidx(e & 255, e >> 8)] = (T)v[m];
    }
}

__host__ __device__ constexpr size_t large_fwd_lds_bytes() {
    return (size_t)4 * kLarge * kLR + (size_t)8 * kLarge * kLR;
}
constexpr int kLargeGS = 64 + 4;  // row stride (floats) of a wave's gradient-tile buffer
__host__ __device__ constexpr size_t large_bwd_lds_bytes() {
    return (size_t)4 * kLarge * kLR + (size_t)8 * kLarge * kLR + (size_t)8 * kLarge * kLR +
           (size_t)8 * 3 * kLarge + (size_t)8 * kLarge * kLR + (size_t)4 * 4 * 16 * kLargeGS;
}

// 4 consecutive floats row[col .. col+3] of a row with `width` valid columns
// (zero beyond; the whole float4 is zero when `ok` is false).
__device__ __forceinline__ float4 load4_masked(const float* row, int col, int width, bool ok) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!ok || col >= width) return v;
    const float* p = row + col;
    if (col + 4 <= width && (reinterpret_cast<uintptr_t>(p) & 15) == 0) return *reinterpret_cast<const float4*>(p);
    v.x = p[0];
    if (col + 1 < width) v.y = p[1];
    if (col + 2 < width) v.z = p[2];
    if (col + 3 < width) v.w = p[3];
    return v;
}
__device__ __forceinline__ float f4_get(const float4& v, int c) {
    return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// Stage rows r0..r0+15 of a [rows][width] matrix (row stride `stride` floats)
// into a swizzled [256][16] LDS array, transposed; zero outside the matrix.
template <typename T>
__device__ __forceinline__ void stage_t(T* dst, const float* src, long long stride, long long r0, long long B,
                                        int width, int t) {
#pragma unroll 4
    for (int m = 0; m < kLR; ++m) {
        const int e = t + kThreads * m;
        const int rr = e >> 8, j = e & 255;
        const long long b = r0 + rr;
        const float v = (b < B && j < width) ? src[b * stride + j] : 0.f;
        dst[zidx(j, rr)] = (T)v;
    }
}

// D[i][r] += sum_j [W_in | W_rec][i][j] * Z[j][r] for the wave's four 16-unit
// blocks (units (4*wave + tb)*16 ..), Z = [zx ; zh].  Chunk (jq, cc) of half g
// and k-slot s contracts j = 256*g + 16*jq + 4*s + cc: one float4 load gives a
// lane its weights for the four chunks of a jq, the four k-slots of a row read
// 64 contiguous bytes, every cache line is consumed within two jq, and every
// chunk reads only one of zx / zh.
// FULL: n_in == n_hid == 256 and 16-byte aligned weights, so the weight loads
// are plain float4 loads with no masking.
template <bool FULL>
__device__ __forceinline__ void large_preact(dbl4 acc[4], const float* __restrict__ w_in,
                                             const float* __restrict__ w_rec, int n_in, int H,
                                             const float* zx, const double* zh, int wave, int lane) {
    const int s = lane >> 4, r = lane & 15;
    dbl4 acc_odd[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc_odd[tb] = dbl4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
    for (int g = 0; g < 2; ++g) {
        const int width = g == 0 ? n_in : H;
        const float* wbase = g == 0 ? w_in : w_rec;
        const float* wrow[4];
        bool rok[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int i = lunit(wave, tb, lane & 15);
            rok[tb] = i < H;
            wrow[tb] = wbase + (long long)min(i, H - 1) * width;
        }
        // FULL: buffer loads from the matrix's descriptor (scalar base), the
        // lane's row and column in the vector offset, the chunk group's
        // column in the scalar offset
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(wbase), (short)0, kLarge * kLarge * 4, kBufferRsrcWord3);
        int voff[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) voff[tb] = lunit(wave, tb, lane & 15) * kLarge * 4;
        auto wload = [&](int tb, int col) -> float4 {
            if constexpr (FULL) {
                const int cs = __builtin_amdgcn_readfirstlane(col - 4 * s);  // the chunk group's first column
                return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[tb] + 16 * s, cs * 4, 0));
            } else {
                return load4_masked(wrow[tb], col, width, rok[tb]);
            }
        };
        float4 w4[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) w4[tb] = wload(tb, 4 * s);
#pragma unroll 2
        for (int jq = 0; jq < 16; ++jq) {
            float4 nw4[4];
            const int jn = jq + 1 < 16 ? jq + 1 : jq;  // prefetch the next chunk group
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) nw4[tb] = wload(tb, 16 * jn + 4 * s);
            double bz[4], wa[4][4];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int jl = 16 * jq + 4 * s + cc;
                bz[cc] = g == 0 ? (double)zx[zidx(jl, r)] : zh[zidx(jl, r)];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) wa[cc][tb] = (double)f4_get(w4[tb], cc);
            }
            // even chunks into acc, odd chunks into acc_odd: a dependent MFMA
            // is always eight issues behind its predecessor
#pragma unroll
            for (int cc = 0; cc < 4; cc += 2) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma_f64(wa[cc][tb], bz[cc], acc[tb]);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc_odd[tb] = mfma_f64(wa[cc + 1][tb], bz[cc + 1], acc_odd[tb]);
            }
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) w4[tb] = nw4[tb];
        }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] += acc_odd[tb];
}

// PARK (one-call entry, overwrite mode): a_k of row b is also written, as
// float64, to a_park + b * N (floats [0, 2 K H) of the row's scratch, which the
// backward overwrites only after reading them back), so the backward needs no
// recomputation.  a_park + b * N must be 8-byte aligned.
template <bool FULL, bool PARK>
__global__ __launch_bounds__(kThreads) void cfc_fwd_large_kernel(
    const float* __restrict__ w_in, const float* __restrict__ w_rec,
    const float* __restrict__ bias, const float* __restrict__ w_tau,
    const float* __restrict__ x, const float* __restrict__ h0, double dt, int B, int K, int n_in,
    int H, float* __restrict__ h_seq, int cell, float* __restrict__ a_park, long long N) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* zx = reinterpret_cast<float*>(smem);                        // [256][16] x_k
    double* zh = reinterpret_cast<double*>(smem + 4 * kLarge * kLR);   // [256][16] h_k
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int s = lane >> 4, r = lane & 15;
    const long long r0 = (long long)blockIdx.x * kLR;

    // this lane's 16 accumulator elements: unit (4*wave + tb)*16 + s + 4v, row r
    double bias_v[4][4], spdt_v[4][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = lunit(wave, tb, s + 4 * v);
            bias_v[tb][v] = i < H ? (double)bias[i] : 0.0;
            // gated: softplus(w_tau) dt; tau-decay: the decay itself
            double decay = 0.0, q;
            if (cell == CFC_CELL_TAU_DECAY && i < H) tau_decay_consts((double)w_tau[i], dt, decay, q);
            spdt_v[tb][v] = i >= H ? 0.0 : cell == CFC_CELL_TAU_DECAY ? decay : softplus_f64((double)w_tau[i]) * dt;
        }
    stage_t(zh, h0, H, r0, B, H, t);
    stage_t(zx, x, (long long)K * n_in, r0, B, n_in, t);
    __syncthreads();

    for (int k = 0; k < K; ++k) {
        dbl4 acc[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[tb] = dbl4{0.0, 0.0, 0.0, 0.0};
        large_preact<FULL>(acc, w_in, w_rec, n_in, H, zx, zh, wave, lane);
        // next step's inputs, loaded after the product's weight loads (so
        // that their in-order waits do not cover these) and written to LDS
        // after the elementwise phase
        float xn[kLR];
#pragma unroll
        for (int m = 0; m < kLR; ++m) {
            const int e = t + kThreads * m;
            const int rr = e >> 8, j = e & 255;
            const long long b = r0 + rr;
            xn[m] = (k + 1 < K && b < B && j < n_in) ? x[(b * K + k + 1) * (long long)n_in + j] : 0.f;
        }
        __syncthreads();  // every wave is done reading zx / zh of step k
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            // the four units' states first: read after a store to zh, each
            // unit's read would wait for the previous unit's store
            double hv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) hv[v] = zh[zidx(lunit(wave, tb, s + 4 * v), r)];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = lunit(wave, tb, s + 4 * v);
                const double a = acc[tb][v] + bias_v[tb][v];
                if constexpr (PARK) {
                    if (r0 + r < B && i < H)
                        reinterpret_cast<double*>(a_park + (r0 + r) * N)[(long long)k * H + i] = a;
                }
                const double g = cell == CFC_CELL_TAU_DECAY
                                     ? spdt_v[tb][v]
                                     : inv_one_plus_exp_exact(spdt_v[tb][v], spdt_v[tb][v] * kLog2e, a);
                const double c = fma(-2.0, inv_one_plus_exp_exact(2.0, 2.0 * kLog2e, a), 1.0);
                zh[zidx(i, r)] = fma(g, hv[v] - c, c);  // g*h + (1-g)*c
            }
        }
#pragma unroll
        for (int m = 0; m < kLR; ++m) {
            const int e = t + kThreads * m;
            zx[zidx(e & 255, e >> 8)] = xn[m];
        }
        __syncthreads();
        // h_k+1 of the 16 rows, row-contiguous stores
#pragma unroll 4
        for (int m = 0; m < kLR; ++m) {
            const int e = t + kThreads * m;
            const int rr = e >> 8, j = e & 255;
            const long long b = r0 + rr;
            if (b < B && j < H) h_seq[(b * K + k) * (long long)H + j] = (float)zh[zidx(j, rr)];
        }
    }
}

// The one-call path at exactly 256 x 256 reads its weights as float64 when
// B >= 4: a short kernel widens [W_in ; W_rec] once per call into the middle
// of scratch rows 0..3, which no other kernel of the call touches before the
// weight-gradient phase rewrites those rows.  Quarter q (row q, floats
// [off, off + 65536) with off = 2 K H, between the parked values in the head
// and the dL/dw_tau sums in the last 2 H floats) holds unit rows 128 (q & 1) .. 128 (q & 1) +
// 127 of W_in (q < 2) or W_rec (q >= 2), row-major, in float64.  The
// products then need no float32 -> float64 conversion per operand; vector
// instructions stall the f64 matrix cores of their SIMD (measured on MI355X:
// the forward 0.43 -> 0.41 ms and phase 1 0.30 -> 0.28 ms at B = 8192, K = 8).
constexpr long long kWideElems = 2LL * kLarge * kLarge;
__global__ __launch_bounds__(kThreads) void widen_weights_kernel(const float* __restrict__ w_in,
                                                                 const float* __restrict__ w_rec,
                                                                 float* __restrict__ wide, long long N) {
    const int e = blockIdx.x * kThreads + threadIdx.x;  // grid: kWideElems / kThreads
    const int g = e >> 16, u = (e >> 8) & 255, j = e & 255;
    const float v = g == 0 ? w_in[e & 65535] : w_rec[e & 65535];
    reinterpret_cast<double*>(wide + (long long)(2 * g + (u >> 7)) * N)[(u & 127) * kLarge + j] = (double)v;
}
// a quarter of the copy: 128 unit rows of 256 doubles
constexpr int kWideQuarterBytes = 128 * kLarge * 8;
constexpr long long kWideQuarterFloats = kWideQuarterBytes / 4;
// four consecutive weights of one unit row, as the products take them
struct W4f {
    float4 v;
    __device__ double get(int cc) const { return (double)f4_get(v, cc); }
};
struct W4d {
    double2 lo, hi;
    __device__ double get(int cc) const { return cc == 0 ? lo.x : cc == 1 ? lo.y : cc == 2 ? hi.x : hi.y; }
};

// Thirty-two rows per workgroup, for exactly 256 x 256 with 16-byte-aligned
// weights.  Each weight operand (a float4 load and its widening) then feeds
// the products of two 16-row tiles, so the widenings per matrix-core product
// halve against cfc_fwd_large_kernel; f64 matrix-core products and vector
// instructions do not overlap on a SIMD (measured on MI355X: each vector
// instruction between two products adds 13 cycles or more), so the widenings
// set the product loop's pace.  [x_k ; h_k] of the 32 rows is staged as in
// the 16-row kernel, in [256][32] arrays swizzled within each row of 32.
// PARK as in cfc_fwd_large_kernel: a_k of row b goes to a_park + b N, with
// N the scratch row length (overwrite mode) or 2 K H (the caller's workspace
// in accumulate mode).  W64: the weights come from the widened float64 copy
// `wide`, its quarters wstride floats apart (see widen_weights_kernel: in
// scratch rows 0..3 in overwrite mode, after the parks in the workspace in
// accumulate mode).
constexpr int kLR2 = 32;  // batch rows per workgroup of the 32-row forward
__device__ __forceinline__ int zidx2(int j, int r) { return j * kLR2 + (r ^ (j & 31)); }
__host__ __device__ constexpr size_t large32_fwd_lds_bytes() {
    return (size_t)4 * kLarge * kLR2 + (size_t)8 * kLarge * kLR2 + (size_t)8 * 2 * kLarge;
}
template <bool PARK, bool W64>
__global__ __launch_bounds__(kThreads) void cfc_fwd_large32_kernel(
    const float* __restrict__ w_in, const float* __restrict__ w_rec, const float* __restrict__ bias,
    const float* __restrict__ w_tau, const float* __restrict__ x, const float* __restrict__ h0, double dt, int B,
    int K, float* __restrict__ h_seq, int cell, float* __restrict__ a_park, long long N,
    const float* __restrict__ wide, long long wstride) {
    constexpr int H = kLarge, NI = kLarge;
    extern __shared__ __align__(16) unsigned char smem[];
    float* zx = reinterpret_cast<float*>(smem);                          // [256][32] x_k
    double* zh = reinterpret_cast<double*>(smem + 4 * kLarge * kLR2);     // [256][32] h_k
    double* ubias = reinterpret_cast<double*>(smem + 12 * kLarge * kLR2); // [256] b
    double* uspdt = ubias + kLarge;  // [256] softplus(w_tau) dt (tau-decay: the decay)
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int s = lane >> 4, r = lane & 15;
    const long long r0 = (long long)blockIdx.x * kLR2;
    static_assert(kThreads == kLarge, "one thread per unit for the per-unit constants");
    {
        const double w = (double)w_tau[t];
        ubias[t] = (double)bias[t];
        if (cell == CFC_CELL_TAU_DECAY) {
            double decay = 0.0, q;
            tau_decay_consts(w, dt, decay, q);
            uspdt[t] = decay;
        } else {
            uspdt[t] = softplus_f64(w) * dt;
        }
    }
    // h_0 and x_0 of the 32 rows (rows >= B zero)
#pragma unroll 4
    for (int m = 0; m < kLR2; ++m) {
        const int e = t + kThreads * m, rr = e >> 8, j = e & 255;
        const long long b = r0 + rr;
        zh[zidx2(j, rr)] = b < B ? (double)h0[b * H + j] : 0.0;
        zx[zidx2(j, rr)] = b < B ? x[b * K * (long long)NI + j] : 0.f;
    }
    __syncthreads();

    for (int k = 0; k < K; ++k) {
        // D[i][r] = sum_j [W_in | W_rec][i][j] [x_k ; h_k][j][r] for the
        // wave's four 16-unit tiles and both 16-row tiles; chunk (jq, cc) of
        // half g and k-slot s contracts j = 256 g + 16 jq + 4 s + cc (the
        // 16-row kernel's order), eight independent accumulators per chunk
        dbl4 acc[4][2];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) acc[tb][rt] = dbl4{0.0, 0.0, 0.0, 0.0};
        // both halves unrolled, so that the operand array of each is fixed
        // at compile time (no per-read branch), and the swizzled operand
        // offsets of the lane precomputed: chunk j = 32 jp + jr reads element
        // 1024 jp + off[jr's parity][cc][rt], jr = 16 (jq & 1) + 4 s + cc
        int off[2][4][2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) off[p][cc][rt] = zidx2(16 * p + 4 * s + cc, 16 * rt + r);
        // half g of the contraction; load(tb, jq) gives the four weights of
        // chunk group jq for tile tb (float32 or the widened float64 copy)
        auto half = [&](const int g, auto load) {
            decltype(load(0, 0)) w4[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) w4[tb] = load(tb, 0);
            // eight chunk groups per loop trip: the LDS operand offsets of the
            // trip's groups are immediates (0.354 against 0.365 ms with four;
            // all sixteen spill registers)
#pragma unroll 8
            for (int jq = 0; jq < 16; ++jq) {
                decltype(load(0, 0)) nw4[4];
                const int jn = jq + 1 < 16 ? jq + 1 : jq;  // the next chunk group's weights
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) nw4[tb] = load(tb, jn);
                const int base = 1024 * (jq >> 1), par = jq & 1;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    double bz[2];
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
                        bz[rt] = g == 0 ? (double)zx[base + off[par][cc][rt]] : zh[base + off[par][cc][rt]];
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        const double wa = w4[tb].get(cc);
#pragma unroll
                        for (int rt = 0; rt < 2; ++rt) acc[tb][rt] = mfma_f64(wa, bz[rt], acc[tb][rt]);
                    }
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) w4[tb] = nw4[tb];
            }
        };
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            if constexpr (W64) {
                // the wave's units 64 wave .. 64 wave + 63 lie in one quarter of
                // the copy: one buffer descriptor per wave (its base in scalar
                // registers), a lane offset per tile, and each load's
                // chunk-group offset as the instruction's immediate.  Measured
                // on MI355X against the same loads through 64-bit addresses:
                // 0.37 against 0.41 ms for the forward at B = 8192.
                const int wq = __builtin_amdgcn_readfirstlane(wave);
                const __amdgpu_buffer_rsrc_t rs =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(wide + (long long)(2 * g + (wq >> 1)) * wstride),
                                                      (short)0, kWideQuarterBytes, kBufferRsrcWord3);
                int voff[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) voff[tb] = ((lunit(wave, tb, r) & 127) * kLarge + 4 * s) * 8;
                half(g, [&](int tb, int jq) {
                    const auto lo = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[tb] + 128 * jq, 0, 0);
                    const auto hi = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[tb] + 128 * jq + 16, 0, 0);
                    return W4d{__builtin_bit_cast(double2, lo), __builtin_bit_cast(double2, hi)};
                });
            } else {
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float*>(g == 0 ? w_in : w_rec), (short)0, kLarge * kLarge * 4, kBufferRsrcWord3);
                int voff[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) voff[tb] = (lunit(wave, tb, r) * kLarge + 4 * s) * 4;
                half(g, [&](int tb, int jq) {
                    return W4f{__builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[tb], 64 * jq, 0))};
                });
            }
        }
        // next step's x, loaded after the product's weight loads and written
        // to LDS after the elementwise phase
        float xn[kLR2];
#pragma unroll
        for (int m = 0; m < kLR2; ++m) {
            const int e = t + kThreads * m, rr = e >> 8, j = e & 255;
            const long long b = r0 + rr;
            xn[m] = (k + 1 < K && b < B) ? x[(b * K + k + 1) * (long long)NI + j] : 0.f;
        }
        __syncthreads();  // every wave is done reading zx / zh of step k
        // a lane's four tiles hold units 4 m + tb (tb = 0..3) of a row: four
        // consecutive doubles of its parked a_k, stored as two 16-byte
        // halves, so the four k-slots of a row fill whole 128-byte lines
        // (one 8-byte store per value wrote twice the bytes to HBM)
        const bool park_vec = (reinterpret_cast<uintptr_t>(a_park) & 15) == 0;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int rr = 16 * rt + r;
                double av[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) av[tb] = acc[tb][rt][v] + ubias[lunit(wave, tb, s + 4 * v)];
                if constexpr (PARK) {
                    if (r0 + rr < B) {
                        double* dst = reinterpret_cast<double*>(a_park + (r0 + rr) * N) + (long long)k * H +
                                      lunit(wave, 0, s + 4 * v);
                        if (park_vec) {
                            reinterpret_cast<double2*>(dst)[0] = make_double2(av[0], av[1]);
                            reinterpret_cast<double2*>(dst)[1] = make_double2(av[2], av[3]);
                        } else {
#pragma unroll
                            for (int tb = 0; tb < 4; ++tb) dst[tb] = av[tb];
                        }
                    }
                }
                // the four units' LDS operands first: read after a store to
                // zh, each unit's reads waited for the previous unit's store
                // (forward at B = 8192: 0.355 -> 0.348 ms; evaluating the
                // four units' exponentials step by step side by side gained
                // nothing more: this phase is bound by its f64 issue)
                double sp[4], hv[4], c[4], gt[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const int i = lunit(wave, tb, s + 4 * v);
                    sp[tb] = uspdt[i];
                    hv[tb] = zh[zidx2(i, rr)];
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) c[tb] = fma(-2.0, inv_one_plus_exp_exact(2.0, 2.0 * kLog2e, av[tb]), 1.0);
                if (cell == CFC_CELL_TAU_DECAY) {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) gt[tb] = sp[tb];
                } else {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) gt[tb] = inv_one_plus_exp_exact(sp[tb], sp[tb] * kLog2e, av[tb]);
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    hv[tb] = fma(gt[tb], hv[tb] - c[tb], c[tb]);  // g*h + (1-g)*c
                    zh[zidx2(lunit(wave, tb, s + 4 * v), rr)] = hv[tb];
                }
            }
#pragma unroll
        for (int m = 0; m < kLR2; ++m) {
            const int e = t + kThreads * m;
            zx[zidx2(e & 255, e >> 8)] = xn[m];
        }
        __syncthreads();
        // h_k+1 of the 32 rows, row-contiguous stores
#pragma unroll 4
        for (int m = 0; m < kLR2; ++m) {
            const int e = t + kThreads * m, rr = e >> 8, j = e & 255;
            const long long b = r0 + rr;
            if (b < B) h_seq[(b * K + k) * (long long)H + j] = (float)zh[zidx2(j, rr)];
        }
    }
}

// PARKED (one-call entry, after cfc_fwd_large_kernel<FULL, true>): a_k is read
// back from the head of the row's scratch instead of being recomputed, so x_k
// is not staged; the window is then the whole sequence.
// STAGE 0 runs both phases.  The parked path runs them as two launches, so
// that each gets the compiler's register allocation to itself: STAGE 1 runs
// phase 1, parks each dL/da_k over the a_k it has consumed and leaves each
// row's dL/dw_tau sums (float64) in the last 2 H floats of its scratch row;
// STAGE 2 runs phase 2 and reads both back before the row's gradient
// overwrites them.
// ACC (accumulate mode, STAGE 0, not PARKED): the scratch rows are read and
// the gradient, rounded to float32, is added in float32; dL/da is parked in
// the caller's workspace `ws` (2 K H 32-bit words per row) instead of the
// scratch tail, whose old values are still needed.
// ACC with STAGE 1 (accumulate mode at exactly 256 x 256, K <= 8): dL/da_k is
// parked in `ws` (the same 2 K H words per row, rows back to back; PARKED:
// over the a_k the forward parked there), and each row's dL/dw_tau, rounded
// to float32, is added to its scratch element at once; the weight gradients
// and db follow in cfc_bwd_large_grads_kernel<true>.
// ACC, STAGE 1 without PARKED (cfc_backward accumulating over a whole
// sequence at exactly 256 x 256, K <= 8): phase 1 recomputes a_k as STAGE 0
// does.  In overwrite mode that split measured slower than STAGE 0 (1.48
// against 1.45 ms at B = 8192), in accumulate mode faster (2.29 against 2.53
// ms): there STAGE 0's phase 2 reads the old values on the matrix-core path.
template <bool FULL, bool TAU, bool PARKED, int STAGE = 0, bool ACC = false>
__global__ __launch_bounds__(kThreads) void cfc_bwd_large_kernel(
    const float* __restrict__ w_in, const float* __restrict__ w_rec,
    const float* __restrict__ bias, const float* __restrict__ w_tau,
    const float* __restrict__ x, const float* __restrict__ h0, const float* __restrict__ h_seq,
    const float* __restrict__ y, double dt, int B, BwdWindow win, int n_in, int H, float* __restrict__ scratch,
    float* __restrict__ loss, float* __restrict__ grad_x, unsigned* __restrict__ ws, const float* __restrict__ wide,
    long long wstride) {
    static_assert(!ACC || STAGE != 2, "accumulate mode: both phases in one launch, or phase 1 alone");
    static_assert(PARKED || STAGE == 0 || (ACC && STAGE == 1),
                  "the recomputing kernel runs both phases, or phase 1 alone in accumulate mode");
    constexpr int cell = TAU ? CFC_CELL_TAU_DECAY : CFC_CELL_GATED;
    const int K = win.Kw;  // steps of this launch; indices below are relative to win.k0
    const long long Kf = win.K, k0 = win.k0;
    float* __restrict__ grad_h0 = win.delta_out;
    extern __shared__ __align__(16) unsigned char smem[];
    float* zx = reinterpret_cast<float*>(smem);                             // [256][16] x_k
    double* zh = reinterpret_cast<double*>(smem + 4 * kLarge * kLR);        // [256][16] h_k
    double* dab = reinterpret_cast<double*>(smem + 12 * kLarge * kLR);      // [256][16] dL/da_k
    double* ubias = reinterpret_cast<double*>(smem + 20 * kLarge * kLR);    // [256] per-unit b,
    double* uspdt = ubias + kLarge;  // softplus(w_tau)*dt (tau-decay: the decay),
    double* usw = uspdt + kLarge;    // sigmoid(w_tau) (tau-decay: d decay / d tau / decay)
    double* gwt = usw + kLarge;  // [256][16] dL/dw_tau sums; each element owned by one lane
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int s = lane >> 4, r = lane & 15;
    const long long r0 = (long long)blockIdx.x * kLR;
    const long long N = (long long)H * (n_in + H + 2);
    const long long b_own = r0 + r;
    const bool row_ok = b_own < B;
    // dL/da of every step is parked in its row's scratch (as two 32-bit halves
    // per double) until the row's weight gradients are formed; every element
    // there is rewritten afterwards.  PARKED: in the head, each dL/da_k over
    // the a_k it was formed from (read one step earlier), so the call's parked
    // values occupy one 2 K H-float region per row instead of two and fit the
    // memory-side cache better; recomputing kernels: in the tail.  ACC parks
    // it in ws.
    const long long tmp_off = PARKED ? 0 : N - 2LL * K * H;
    auto park_row = [&](long long b) -> unsigned* {
        if constexpr (ACC) return ws + b * (2LL * K * H);
        else return reinterpret_cast<unsigned*>(scratch + b * N + tmp_off);
    };

    if constexpr (STAGE != 2) {
    for (int u = t; u < kLarge; u += kThreads) {
        const bool ok = u < H;
        const double w = ok ? (double)w_tau[u] : 0.0;
        ubias[u] = ok ? (double)bias[u] : 0.0;
        if (cell == CFC_CELL_TAU_DECAY) {
            double decay = 0.0, q = 0.0;
            if (ok) tau_decay_consts(w, dt, decay, q);
            uspdt[u] = decay;
            usw[u] = q;
        } else {
            uspdt[u] = ok ? softplus_f64(w) * dt : 0.0;
            usw[u] = ok ? logistic_f64(w) : 0.0;
        }
    }
    double delta[4][4];
    double lsum = 0.0;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = lunit(wave, tb, s + 4 * v);
            const bool ok = i < H;
            double d = 0.0;
            if (ok && row_ok)
                d = win.delta_in ? (double)win.delta_in[b_own * H + i]
                                 : (double)h_seq[(b_own * Kf + Kf - 1) * H + i] - (double)y[b_own * H + i];
            delta[tb][v] = d;
            lsum += 0.5 * d * d;
            gwt[zidx(i, r)] = 0.0;
        }
    // loss of each row: lanes r, r+16, r+32, r+48 of every wave share row r
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (lane < 16) dab[wave * 16 + lane] = lsum;
    __syncthreads();
    if (t < kLR && loss && !win.delta_in && r0 + t < B)
        loss[r0 + t] = (float)(((dab[t] + dab[16 + t]) + dab[32 + t]) + dab[48 + t]);

    // inputs of step k (x_k and h_k-1 of the 16 rows), fetched one step ahead
    float xr[kLR], hr[kLR];
    auto fetch_step = [&](int k) {
        if constexpr (!PARKED) fetch_t(xr, x + (k0 + k) * n_in, Kf * n_in, r0, B, n_in, t);
        if (k0 + k == 0) fetch_t(hr, h0, H, r0, B, H, t);
        else fetch_t(hr, h_seq + (k0 + k - 1) * H, Kf * H, r0, B, H, t);
    };
    fetch_step(K - 1);
    // PARKED: a_k of the step to come, fetched during the current step's
    // products (after their weight loads, which in-order waits then skip)
    dbl4 apre[4];
    auto fetch_a = [&](int k) {
        if constexpr (PARKED) {
            const double* ap = reinterpret_cast<const double*>(park_row(b_own)) + (k0 + k) * (long long)H;
            if (FULL && (reinterpret_cast<uintptr_t>(ACC ? static_cast<const void*>(ws) : scratch) & 15) == 0) {
                // units lunit(wave, 0..3, m) are four consecutive doubles
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    double2 lo = make_double2(0.0, 0.0), hi = make_double2(0.0, 0.0);
                    if (row_ok) {
                        const double2* q = reinterpret_cast<const double2*>(ap + lunit(wave, 0, s + 4 * v));
                        lo = q[0];
                        hi = q[1];
                    }
                    apre[0][v] = lo.x;
                    apre[1][v] = lo.y;
                    apre[2][v] = hi.x;
                    apre[3][v] = hi.y;
                }
                return;
            }
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = lunit(wave, tb, s + 4 * v);
                    apre[tb][v] = row_ok && i < H ? ap[i] : 0.0;
                }
        }
    };
    fetch_a(K - 1);
    const int jw = 64 * wave + 4 * (lane & 15);
    // accp += M^T dL/da_k for a weight matrix M (rows: the H units, row
    // stride ld, width columns): chunk ic of k-slot s contracts unit
    // i = 64*s + ic; the four tiles' operands M[i][lunit(wave, 0..3, lane%16)]
    // are one float4.  The float4 operands are double-buffered PF chunks
    // ahead, so their L2 latency hides under the previous chunks' products
    // (PF = 4 where the registers allow it, else 2); the next step's inputs
    // are fetched after the last of them if asked.  With `wide` (FULL phase 1
    // of the parked path) the operands come from the widened float64 copy of
    // M (g = 0: W_in, 1: W_rec) as two double2 loads, with no conversions.
    constexpr int PF = FULL ? 4 : 2;
    auto dab_product = [&](const float* __restrict__ wm, int g, int ld, int width, dbl4 (&accp)[4],
                           bool fetch_next, int k) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) accp[tb] = dbl4{0.0, 0.0, 0.0, 0.0};
        if constexpr (FULL && PARKED && STAGE == 1) {
            if (wide) {
                // chunk ic of k-slot s is unit row i = 64 s + ic: the lane's
                // quarter of the copy is fixed (i >> 7 = s >> 1).  One buffer
                // descriptor spans both quarters of the matrix (quarters 2g
                // and 2g + 1, wstride floats apart); the lane's offset selects
                // its quarter and column, the chunk's row goes in the scalar
                // offset.
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float*>(wide + (long long)(2 * g) * wstride), (short)0,
                    (int)(wstride * 4) + kWideQuarterBytes, kBufferRsrcWord3);
                const int voff = (int)((s >> 1) * wstride * 4) + ((64 * (s & 1)) * kLarge + jw) * 8;
                auto wld64 = [&](int ic) -> W4d {
                    const auto lo = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, ic * kLarge * 8, 0);
                    const auto hi = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, ic * kLarge * 8, 0);
                    return W4d{__builtin_bit_cast(double2, lo), __builtin_bit_cast(double2, hi)};
                };
                auto chunks64 = [&](const W4d (&w)[PF], int icb) {
#pragma unroll
                    for (int u = 0; u < PF; ++u) {
                        const double bz = dab[zidx(64 * s + icb + u, r)];
#pragma unroll
                        for (int q = 0; q < 4; ++q) accp[q] = mfma_f64(w[u].get(q), bz, accp[q]);
                    }
                };
                W4d va[PF], vb[PF];
#pragma unroll
                for (int u = 0; u < PF; ++u) va[u] = wld64(u);
                // two trips per loop iteration (phase 1 at B = 8192: 0.263
                // against 0.274 ms with one; prefetching 2 or 8 chunks instead
                // of 4 measured no better)
#pragma unroll 2
                for (int ic0 = 0; ic0 < 64 - 2 * PF; ic0 += 2 * PF) {
#pragma unroll
                    for (int u = 0; u < PF; ++u) vb[u] = wld64(ic0 + PF + u);
                    chunks64(va, ic0);
#pragma unroll
                    for (int u = 0; u < PF; ++u) va[u] = wld64(ic0 + 2 * PF + u);
                    chunks64(vb, ic0 + PF);
                }
#pragma unroll
                for (int u = 0; u < PF; ++u) vb[u] = wld64(64 - PF + u);
                chunks64(va, 64 - 2 * PF);
                if (fetch_next) {
                    fetch_step(k - 1);
                    fetch_a(k - 1);
                }
                chunks64(vb, 64 - PF);
                return;
            }
        }
        const __amdgpu_buffer_rsrc_t rsm = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(wm), (short)0, kLarge * kLarge * 4, kBufferRsrcWord3);
        auto wld = [&](int ic) -> float4 {
            const int i = 64 * s + ic;
            if constexpr (FULL)  // lane's row 64 s and column jw in the vector offset, ic in the scalar one
                return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rsm, (64 * s * kLarge + jw) * 4, ic * kLarge * 4, 0));
            else return load4_masked(wm + (long long)min(i, H - 1) * ld, jw, width, i < H);
        };
        auto chunks1 = [&](const float4 (&w4)[1], int icb) {
            const double bz = dab[zidx(64 * s + icb, r)];
            accp[0] = mfma_f64((double)w4[0].x, bz, accp[0]);
            accp[1] = mfma_f64((double)w4[0].y, bz, accp[1]);
            accp[2] = mfma_f64((double)w4[0].z, bz, accp[2]);
            accp[3] = mfma_f64((double)w4[0].w, bz, accp[3]);
        };
        auto chunks = [&](const float4 (&w4)[PF], int icb) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const double bz = dab[zidx(64 * s + icb + u, r)];
                accp[0] = mfma_f64((double)w4[u].x, bz, accp[0]);
                accp[1] = mfma_f64((double)w4[u].y, bz, accp[1]);
                accp[2] = mfma_f64((double)w4[u].z, bz, accp[2]);
                accp[3] = mfma_f64((double)w4[u].w, bz, accp[3]);
            }
        };
        if constexpr (!PARKED) {
            // the recomputing kernels have no registers to spare: plain
            // loop, the next step's inputs first
            if (fetch_next) {
                fetch_step(k - 1);
                fetch_a(k - 1);
            }
#pragma unroll 4
            for (int ic = 0; ic < 64; ++ic) {
                const float4 w1[1] = {wld(ic)};
                chunks1(w1, ic);
            }
            return;
        }
        float4 wa[PF], wb[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) wa[u] = wld(u);
#pragma unroll 1
        for (int ic0 = 0; ic0 < 64 - 2 * PF; ic0 += 2 * PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) wb[u] = wld(ic0 + PF + u);
            chunks(wa, ic0);
#pragma unroll
            for (int u = 0; u < PF; ++u) wa[u] = wld(ic0 + 2 * PF + u);
            chunks(wb, ic0 + PF);
        }
        // the last block, with the next step's fetch after its weight loads
#pragma unroll
        for (int u = 0; u < PF; ++u) wb[u] = wld(64 - PF + u);
        chunks(wa, 64 - 2 * PF);
        if (fetch_next) {
            fetch_step(k - 1);
            fetch_a(k - 1);
        }
        chunks(wb, 64 - PF);
    };
    for (int k = K - 1; k >= 0; --k) {
        dbl4 acc[4];  // a_k - b (recomputed), or a_k itself (parked)
        if constexpr (PARKED) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc[tb] = apre[tb];
        }
        __syncthreads();  // previous step is done with zx, zh, dab
        if constexpr (!PARKED) store_t(zx, xr, t);
        store_t(zh, hr, t);
        __syncthreads();
        if constexpr (!PARKED) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc[tb] = dbl4{0.0, 0.0, 0.0, 0.0};
            large_preact<FULL>(acc, w_in, w_rec, n_in, H, zx, zh, wave, lane);
        }
        double gk[4][4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                // the four units' LDS operands first: read after the stores
                // to gwt and dab, each unit's reads would wait for the
                // previous unit's stores
                double spv[4], swv[4], hpv[4], gwv[4], bv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = lunit(wave, tb, s + 4 * v);
                    spv[v] = uspdt[i];
                    swv[v] = usw[i];
                    hpv[v] = zh[zidx(i, r)];
                    gwv[v] = gwt[zidx(i, r)];
                    bv[v] = PARKED ? 0.0 : ubias[i];
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = lunit(wave, tb, s + 4 * v);
                    const double spdt = spv[v];
                    const double a = PARKED ? acc[tb][v] : acc[tb][v] + bv[v];
                    const double c = fma(-2.0, inv_one_plus_exp_exact(2.0, 2.0 * kLog2e, a), 1.0);
                    const double hp = hpv[v];
                    const double d = delta[tb][v];
                    double g, da;
                    if constexpr (TAU) {
                        g = spdt;
                        const double dg = d * (hp - c);  // dL/d(decay)
                        da = d * (1.0 - g) * (1.0 - c * c);
                        gwt[zidx(i, r)] = gwv[v] + dg * g * swv[v];
                    } else {
                        g = inv_one_plus_exp_exact(spdt, spdt * kLog2e, a);
                        const double dz = d * (hp - c) * g * (1.0 - g);
                        da = d * (1.0 - g) * (1.0 - c * c) - dz * spdt;
                        gwt[zidx(i, r)] = gwv[v] + dz * (-a * dt) * swv[v];
                    }
                    gk[tb][v] = g;
                    dab[zidx(i, r)] = da;
                }
            }
        __syncthreads();  // dab of step k complete
        if (k > 0 || grad_h0) {
            // delta_k = delta_k+1 * g + W_rec^T dL/da
            dbl4 acc2[4];
            dab_product(w_rec, 1, H, H, acc2, k > 0 && !grad_x, k);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    delta[tb][v] = fma(delta[tb][v], gk[tb][v], acc2[tb][v]);
        }
        if (grad_x) {
            // dL/dx_k = W_in^T dL/da, the same product with W_in's rows; the
            // lane's elements are column lunit(wave, tb, s + 4v) of row r
            dbl4 acc3[4];
            dab_product(w_in, 0, n_in, n_in, acc3, k > 0, k);
            if (row_ok) {
                float* gx = grad_x + (b_own * Kf + k0 + k) * n_in;
                if (FULL && (reinterpret_cast<uintptr_t>(grad_x) & 15) == 0) {
                    // columns lunit(wave, 0..3, m) are consecutive: one float4
                    // per m (B = 8192 with input gradients: 1.591 -> 1.574 ms
                    // for the one-call kernels, against 16 scalar stores)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        *reinterpret_cast<f32x4*>(gx + lunit(wave, 0, s + 4 * v)) =
                            f32x4{(float)acc3[0][v], (float)acc3[1][v], (float)acc3[2][v], (float)acc3[3][v]};
                } else {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int j = lunit(wave, tb, s + 4 * v);
                            if (j < n_in) gx[j] = (float)acc3[tb][v];
                        }
                }
            }
        }
        // park dL/da_k of the 16 rows (PARKED: over a_k, in the heads; else in
        // the tails), row-contiguous
        // (after the products, so that their weight loads' waits do not
        // cover these stores)
#pragma unroll 4
        for (int m = 0; m < kLR; ++m) {
            const int e = t + kThreads * m;
            const int rr = e >> 8, i = e & 255;
            const long long b = r0 + rr;
            if (b < B && i < H) {
                const unsigned long long u = __builtin_bit_cast(unsigned long long, dab[zidx(i, rr)]);
                unsigned* q = park_row(b) + 2 * ((long long)k * H + i);
                q[0] = (unsigned)u;
                q[1] = (unsigned)(u >> 32);
            }
        }
    }
    if (grad_h0 && row_ok) {  // after the window's first step, delta is dL/dh_k0
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int j = lunit(wave, tb, s + 4 * v);
                if (j < H) grad_h0[b_own * H + j] = (float)delta[tb][v];
            }
    }
    if constexpr (STAGE == 1) {
        // the rows' dL/dw_tau sums to the last 2 H floats of their scratch
        // rows (accumulate mode: added to the rows' dL/dw_tau elements)
        __syncthreads();
        for (int e = t; e < kLR * kLarge; e += kThreads) {
            const int rr = e / kLarge, u = e % kLarge;
            const long long b = r0 + rr;
            if (b < B && u < H) {
                if constexpr (ACC) scratch[b * N + N - H + u] += (float)gwt[zidx(u, rr)];
                else reinterpret_cast<double*>(scratch + b * N + N - 2LL * H)[u] = gwt[zidx(u, rr)];
            }
        }
        return;
    }
    }  // STAGE != 2

    // ---- per row: G = DA^T [X | H_prev] over the K steps, then db and dw_tau.
    // The float4 gradient stores are non-temporal: at these widths the scratch
    // is gigabytes, written once and streamed next by the reducer.  With
    // ordinary stores the reduce that follows a 4.3 GB backward took 0.87 ms
    // (0.70 ms on the same buffer after any other 512 MB of traffic); with
    // non-temporal ones it takes 0.76-0.79 ms, and the backward itself is no
    // slower (measured on MI355X).
    __syncthreads();
    const int KP = (K + 3) & ~3;
    double* dak = reinterpret_cast<double*>(smem);                       // [KP][256] dL/da
    float* zk = reinterpret_cast<float*>(smem + (size_t)8 * KP * kLarge);  // [KP][512] [x | h_prev]
    float* gst = reinterpret_cast<float*>(smem + large_bwd_lds_bytes() - (size_t)4 * 4 * 16 * kLargeGS) +
                 wave * 16 * kLargeGS;  // this wave's [16][kLargeGS] tile buffer
    // operands of one row, fetched into registers one row ahead: thread t
    // holds dL/da_kk[t] (parked by phase 1), x_kk[t] and h_kk-1[t]
    double pd[kLargeBwdMaxK];
    float px[kLargeBwdMaxK], ph[kLargeBwdMaxK];
    double pg = 0.0;  // STAGE 2: dL/dw_tau of unit t, from the row's last 2 H floats
    auto fetch_row = [&](long long b) {
        if constexpr (STAGE == 2) pg = t < H ? reinterpret_cast<const double*>(scratch + b * N + N - 2LL * H)[t] : 0.0;
        const unsigned* tq = park_row(b);
#pragma unroll
        for (int kk = 0; kk < kLargeBwdMaxK; ++kk) {
            double dv = 0.0;
            float xv = 0.f, hv = 0.f;
            if (kk < K) {
                if (t < H) {
                    const long long q = 2 * ((long long)kk * H + t);
                    dv = __builtin_bit_cast(double, ((unsigned long long)tq[q + 1] << 32) | tq[q]);
                    hv = k0 + kk == 0 ? h0[b * H + t] : h_seq[(b * Kf + k0 + kk - 1) * H + t];
                }
                if (t < n_in) xv = x[(b * Kf + k0 + kk) * n_in + t];
            }
            pd[kk] = dv;
            px[kk] = xv;
            ph[kk] = hv;
        }
    };
    fetch_row(r0);  // r0 < B: the grid has no empty workgroup
    for (int rr = 0; rr < kLR; ++rr) {
        const long long b = r0 + rr;
        if (b >= B) break;
        const double gw_t = pg;
#pragma unroll
        for (int kk = 0; kk < kLargeBwdMaxK; ++kk) {
            if (kk < KP) {
                dak[kk * kLarge + t] = pd[kk];
                zk[kk * 2 * kLarge + t] = px[kk];
                zk[kk * 2 * kLarge + kLarge + t] = ph[kk];
            }
        }
        __syncthreads();
        if (rr + 1 < kLR && b + 1 < B) fetch_row(b + 1);
        float* grow = scratch + b * N;
        float* grec = grow + (long long)H * n_in;
        // the wave's 64 units x 512 columns: per 64-column group, the four
        // 16-unit tiles together (16 accumulators, so each operand fetched
        // from LDS feeds four MFMAs and a group runs 16 KP/4 of them), then
        // each 16 x 64 tile transposed through LDS into float4 row stores.
        // The dL/da operands of the wave's tiles are read once per row.
        constexpr int KCM = kLargeBwdMaxK / 4;
        const int KC = KP / 4;
        double av[KCM][4];
#pragma unroll
        for (int kc = 0; kc < KCM; ++kc)
#pragma unroll
            for (int ub = 0; ub < 4; ++ub)
                av[kc][ub] = kc < KC ? dak[(4 * kc + s) * kLarge + (4 * wave + ub) * 16 + (lane & 15)] : 0.0;
        if constexpr (FULL && PARKED) {
            // 256 x 256 with aligned rows: no masking, and the work runs as
            // (column group, pair of 16-unit tiles) steps whose two tiles are
            // stored (held in float32 registers) under the first chunk's
            // products of the next step
            const int c4 = 4 * (lane & 15);
            float pend[2][4][4];
            auto store_tiles = [&](int jgp, int uhp) {
#pragma unroll
                for (int u2 = 0; u2 < 2; ++u2) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            gst[(s + 4 * v) * kLargeGS + jj * 16 + (lane & 15)] = pend[u2][jj][v];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int rr2 = s + 4 * m;
                        const float4 val = *reinterpret_cast<const float4*>(gst + rr2 * kLargeGS + c4);
                        const int i = (4 * wave + 2 * uhp + u2) * 16 + rr2;
                        const int jc0 = jgp * 64 + c4;
                        float* dst = jc0 < kLarge ? grow + (long long)i * kLarge + jc0
                                                  : grec + (long long)i * kLarge + (jc0 - kLarge);
                        store_stream_f32x4(dst, f32x4{val.x, val.y, val.z, val.w});
                    }
                }
            };
            for (int jg = 0; jg < 2 * kLarge / 64; ++jg) {
#pragma unroll
                for (int uh = 0; uh < 2; ++uh) {
                    dbl4 acc2[2][4];
#pragma unroll
                    for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) acc2[u2][jj] = dbl4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
                    for (int kc = 0; kc < KCM; ++kc) {
                        if (kc == 0 || kc < KC) {
                            const int kk = 4 * kc + s;
                            double z[4];
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj)
                                z[jj] = (double)zk[kk * 2 * kLarge + (4 * jg + jj) * 16 + (lane & 15)];
#pragma unroll
                            for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
                                    acc2[u2][jj] = mfma_f64(av[kc][2 * uh + u2], z[jj], acc2[u2][jj]);
                            if (kc == 0) {
                                if (uh == 1) store_tiles(jg, 0);
                                else if (jg > 0) store_tiles(jg - 1, 1);
                            }
                        }
                    }
#pragma unroll
                    for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                            for (int v = 0; v < 4; ++v) pend[u2][jj][v] = (float)acc2[u2][jj][v];
                }
            }
            store_tiles(2 * kLarge / 64 - 1, 1);
        }
        for (int jg = 0; jg < (FULL && PARKED ? 0 : 2 * kLarge / 64); ++jg) {
            dbl4 acc4[4][4];
#pragma unroll
            for (int ub = 0; ub < 4; ++ub)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc4[ub][jj] = dbl4{0.0, 0.0, 0.0, 0.0};
            // ACC: the old float4 values of one 16-unit tile's stores: tile 0's
            // are loaded before the products (their latency hides under
            // them), tile ub + 1's as soon as tile ub is stored (unaligned or
            // partial spans are read at the store instead)
            float4 old[4];
            auto load_old = [&](int ub) {
                if constexpr (ACC) {
                    const int jc0 = jg * 64 + 4 * (lane & 15);
                    const bool in_part = jc0 < kLarge;
                    const int col = in_part ? jc0 : jc0 - kLarge;
                    const int width = in_part ? n_in : H;
                    const float* base = in_part ? grow : grec;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int i = (4 * wave + ub) * 16 + s + 4 * m;
                        const float* src = base + (long long)i * width + col;
                        const bool fast =
                            i < H && col + 4 <= width && (reinterpret_cast<uintptr_t>(src) & 15) == 0;
                        old[m] = fast ? *reinterpret_cast<const float4*>(src) : float4{0.f, 0.f, 0.f, 0.f};
                    }
                }
            };
            load_old(0);
#pragma unroll
            for (int kc = 0; kc < KCM; ++kc) {
                if (kc < KC) {
                    const int kk = 4 * kc + s;
                    double z[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) z[jj] = (double)zk[kk * 2 * kLarge + (4 * jg + jj) * 16 + (lane & 15)];
#pragma unroll
                    for (int ub = 0; ub < 4; ++ub)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) acc4[ub][jj] = mfma_f64(av[kc][ub], z[jj], acc4[ub][jj]);
                }
            }
#pragma unroll
            for (int ub = 0; ub < 4; ++ub) {
                const int ib = 4 * wave + ub;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        gst[(s + 4 * v) * kLargeGS + jj * 16 + (lane & 15)] = (float)acc4[ub][jj][v];
                const int c4 = 4 * (lane & 15);
                const int jc0 = jg * 64 + c4;
                const bool in_part = jc0 < kLarge;
                const int col = in_part ? jc0 : jc0 - kLarge;
                const int width = in_part ? n_in : H;
                float* base = in_part ? grow : grec;
                if constexpr (ACC) {
                    // the tile's sums first, then the next tile's old values
                    // (issued ahead of this tile's stores, so that their wait
                    // does not include the stores' completion), then the stores
                    f32x4 sum[4];
                    float4 tile[4];  // the bare tile, for unaligned or partial spans
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        tile[m] = *reinterpret_cast<const float4*>(gst + (s + 4 * m) * kLargeGS + c4);
                        sum[m] = f32x4{old[m].x + tile[m].x, old[m].y + tile[m].y, old[m].z + tile[m].z,
                                       old[m].w + tile[m].w};
                    }
                    if (ub < 3) load_old(ub + 1);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int i = ib * 16 + s + 4 * m;
                        if (i < H) {
                            float* dst = base + (long long)i * width + col;
                            if (col + 4 <= width && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                                // read-modify-write of the old value: plain
                                // non-temporal store (measured faster here
                                // than the write-through form, 2.98 against
                                // 3.30 ms per large-batch backward)
                                __builtin_nontemporal_store(sum[m], reinterpret_cast<f32x4*>(dst));
                            } else {
                                const float v4[4] = {tile[m].x, tile[m].y, tile[m].z, tile[m].w};
#pragma unroll
                                for (int c = 0; c < 4; ++c)
                                    if (col + c < width) dst[c] += v4[c];
                            }
                        }
                    }
                } else {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int rr2 = s + 4 * m;
                    const float4 val = *reinterpret_cast<const float4*>(gst + rr2 * kLargeGS + c4);
                    const int i = ib * 16 + rr2;
                    if (i < H) {
                        float* dst = base + (long long)i * width + col;
                        if (col + 4 <= width && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                            store_stream_f32x4(dst, f32x4{val.x, val.y, val.z, val.w});
                        } else {
                            if (col < width) dst[0] = val.x;
                            if (col + 1 < width) dst[1] = val.y;
                            if (col + 2 < width) dst[2] = val.z;
                            if (col + 3 < width) dst[3] = val.w;
                        }
                    }
                }
                }
            }
        }
        // db: the row's parked dL/da summed over k, last step first (the order
        // of the per-step accumulation); dw_tau from the lane-owned LDS sums
        if (t < H) {
            double gb = 0.0;
            for (int kk = K - 1; kk >= 0; --kk) gb += dak[kk * kLarge + t];
            if constexpr (ACC) {
                grec[(long long)H * H + t] += (float)gb;
                grec[(long long)H * H + H + t] += (float)gwt[zidx(t, rr)];
            } else {
                grec[(long long)H * H + t] = (float)gb;
                grec[(long long)H * H + H + t] = STAGE == 2 ? (float)gw_t : (float)gwt[zidx(t, rr)];
            }
        }
        __syncthreads();  // LDS reused by the next row
    }
}

// Phase 2 of the parked backward at exactly 256 x 256 and K <= 8, on the
// vector units: one workgroup per row.  The row's weight gradient is a sum of
// K outer products, G[i][j] = sum_k dL/da_k[i] [x_k | h_k-1][j], so each
// output element takes K multiply-adds; as K x 4 f64 FMAs per lane for four
// adjacent columns of one unit row, with the lane's K x 4 operands of
// [x | h_prev] held in registers and the unit's K values of dL/da read from
// LDS as a broadcast, every wave instruction stores 1 KB of contiguous
// gradient.  The matrix-core form of this product (cfc_bwd_large_kernel, the
// other shapes) needs a transpose through LDS per 16 x 64 tile and converts
// its accumulators tile by tile; at K = 8 that measured 0.90 ms for the
// 4.3 GB scratch of B = 8192, of which 0.67 ms without its stores.
// Inputs: dL/da parked in the head of the row's scratch by phase 1 (two 32-bit
// halves per double, [k][unit]) and the dL/dw_tau sums in its last 2 H floats
// (float64); both are read before the barrier that precedes the first store.
// The launch reserves kGradsLdsReserve bytes of dynamic LDS that the kernel
// never touches: with the 16 KB array below a workgroup then takes more than
// half of a CU's 160 KB, so one row is written per CU at a time (256 rows in
// flight instead of 1,024 at the register-bound four per CU).  Fewer
// concurrent write streams keep HBM busier: 0.84 -> 0.81 ms for the 4.3 GB
// of B = 8192, bitwise the same (two or three per CU measured 0.83 ms; a
// persistent grid of 256 workgroups looping over rows, 0.84 ms).
// ACC (accumulate mode, after the parked phase 1 of the one-call entry or the
// recomputing one of cfc_backward): dL/da comes from the caller's workspace
// `ws` (rows of 2 K H words, where phase 1 left it), dL/dw_tau has already been
// added by that phase, and each gradient element, rounded to float32, is added
// to the scratch element in float32.  The old values are read with
// non-temporal loads one block of eight loop trips (16 unit rows) ahead, and
// the sums written through like the overwrite stores.  At B = 8192 this
// kernel moves 8.6 GB: the whole one-call accumulate takes 2.29 ms, against
// 2.93 ms for the forward and the recomputing backward (prefetching two or
// four trips ahead, plain non-temporal stores, or four rows per CU measured
// within 2 % of it).
constexpr int kGradsMaxK = 8;
constexpr size_t kGradsLdsReserve = 68 * 1024;
template <bool ACC>
__global__ __launch_bounds__(kThreads) void cfc_bwd_large_grads_kernel(
    const float* __restrict__ x, const float* __restrict__ h0, const float* __restrict__ h_seq, int K,
    float* __restrict__ scratch, long long N, const unsigned* __restrict__ ws) {
    constexpr int H = kLarge, NI = kLarge;
    __shared__ double das[kLarge][kGradsMaxK];  // dL/da of the row, unit-major
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const long long b = blockIdx.x;
    float* row = scratch + b * N;
    static_assert(kThreads == kLarge, "one thread per unit");
    const unsigned* tq = ACC ? ws + b * (2LL * K * H) : reinterpret_cast<const unsigned*>(row);
    double gb = 0.0;
    for (int kk = K - 1; kk >= 0; --kk) {  // db in the order of the per-step accumulation
        const long long q = 2 * ((long long)kk * H + t);
        const double dv = __builtin_bit_cast(double, ((unsigned long long)tq[q + 1] << 32) | tq[q]);
        das[t][kk] = dv;
        gb += dv;
    }
    for (int kk = K; kk < kGradsMaxK; ++kk) das[t][kk] = 0.0;
    const double gw_t = ACC ? 0.0 : reinterpret_cast<const double*>(row + N - 2LL * H)[t];
    // this lane's four columns of [x_k | h_k-1] for every step: waves 0 and
    // 2 hold x (dW_in), waves 1 and 3 hold h_prev (dW_rec)
    const int part = wave & 1, c = 4 * lane;
    double z[kGradsMaxK][4];
#pragma unroll
    for (int k = 0; k < kGradsMaxK; ++k) {
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (k < K) {
            const float* src = part == 0 ? x + (b * K + k) * NI + c
                                         : (k == 0 ? h0 + b * H + c : h_seq + (b * K + k - 1) * H + c);
            v = *reinterpret_cast<const f32x4*>(src);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) z[k][m] = v[m];
    }
    __syncthreads();  // every read of the row's head and tail precedes every store
    float* base = part == 0 ? row : row + (long long)H * NI;
    // gradient of unit row i for the lane's four columns, float32
    auto grad4 = [&](int i) {
        const double* d = das[i];
        double dk[kGradsMaxK];
#pragma unroll
        for (int k = 0; k < kGradsMaxK; ++k) dk[k] = d[k];
        f32x4 g;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            double a = dk[0] * z[0][m];
#pragma unroll
            for (int k = 1; k < kGradsMaxK; ++k) a = fma(dk[k], z[k][m], a);
            g[m] = (float)a;
        }
        return g;
    };
    if constexpr (ACC) {
        // unit rows i = wave / 2 + 2 u, eight per block of four loop trips;
        // the next block's old values are loaded before this block's products
        constexpr int kTrips = 8;
        f32x4 old[kTrips][2], nxt[kTrips][2];
        auto load_block = [&](int u0, f32x4 (&dst)[kTrips][2]) {
#pragma unroll
            for (int j = 0; j < kTrips; ++j)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int i = (wave >> 1) + 2 * (u0 + 2 * j + p);
                    dst[j][p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + (long long)i * H + c));
                }
        };
        load_block(0, old);
#pragma unroll 1
        for (int u0 = 0; u0 < H / 2; u0 += 2 * kTrips) {
            if (u0 + 2 * kTrips < H / 2) load_block(u0 + 2 * kTrips, nxt);
#pragma unroll
            for (int j = 0; j < kTrips; ++j)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int i = (wave >> 1) + 2 * (u0 + 2 * j + p);
                    store_stream_f32x4(base + (long long)i * H + c, old[j][p] + grad4(i));
                }
            if (u0 + 2 * kTrips < H / 2) {
#pragma unroll
                for (int j = 0; j < kTrips; ++j)
#pragma unroll
                    for (int p = 0; p < 2; ++p) old[j][p] = nxt[j][p];
            }
        }
        // db of unit t (dL/dw_tau was added by phase 1)
        row[(long long)H * (NI + H) + t] += (float)gb;
    } else {
        // unit rows i = wave / 2 + 2 u, two per iteration
#pragma unroll 1
        for (int u = 0; u < H / 2; u += 2) {
            f32x4 g[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) g[p] = grad4((wave >> 1) + 2 * (u + p));
#pragma unroll
            for (int p = 0; p < 2; ++p) store_stream_f32x4(base + (long long)((wave >> 1) + 2 * (u + p)) * H + c, g[p]);
        }
        // db and dw_tau of unit t
        row[(long long)H * (NI + H) + t] = (float)gb;
        row[(long long)H * (NI + H) + H + t] = (float)gw_t;
    }
}

// -------------------------------------------------------- reduce_axis0
// A workgroup (4 waves) owns a tile of TW = LPR * VEC consecutive columns.  A
// row of the tile is read by LPR consecutive lanes (VEC floats each: 256 or
// 512 contiguous bytes per row), so a wave covers 64 / LPR rows per load and
// the workgroup has S = 4 * 64 / LPR row slots.  Slot s sums rows s, s + S,
// s + 2S, ... in that order in float64, with 8 rows' loads in flight; the S
// slot sums of each column are then added in slot order through LDS (rows of
// the LDS array padded by one double).  One float32 store per column.  No
// atomics, so the result is bitwise reproducible.  Every input element is read
// once, so the loads are non-temporal: they stream past the caches instead of
// evicting lines that other work still uses (measured on MI355X: 256-byte row
// segments with non-temporal loads run at 76 % of HBM peak on a 4.3 GB input,
// against 70 % with ordinary loads).
template <int VEC, int LPR>
__global__ __launch_bounds__(kThreads) void reduce_axis0_kernel(const float* __restrict__ in,
                                                                long long B, long long N,
                                                                float* __restrict__ out) {
    constexpr int TW = LPR * VEC;
    constexpr int kRowsPerWave = 64 / LPR;
    constexpr int kSlots = kRowsPerWave * (kThreads / 64);
    constexpr int kUnroll = LPR == 32 ? 16 : 8;
    __shared__ double part[kSlots][TW + 1];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int slot = wave * kRowsPerWave + lane / LPR;
    const int c0 = (lane % LPR) * VEC;  // first column of this lane inside the tile
    const long long col = (long long)blockIdx.x * TW + c0;

    double acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0;

    if (col < N) {  // with VEC == 4, N % 4 == 0, so all 4 columns are in range
        const float* p = in + col;
        long long bb = slot;
        for (; bb + (kUnroll - 1) * kSlots < B; bb += kUnroll * kSlots) {
            if constexpr (VEC == 4) {
                f32x4 q[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    q[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + (bb + u * kSlots) * N));
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    acc[0] += (double)q[u].x;
                    acc[1] += (double)q[u].y;
                    acc[2] += (double)q[u].z;
                    acc[3] += (double)q[u].w;
                }
            } else {
                float q[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) q[u] = __builtin_nontemporal_load(p + (bb + u * kSlots) * N);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) acc[0] += (double)q[u];
            }
        }
        for (; bb < B; bb += kSlots) {
            if constexpr (VEC == 4) {
                const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + bb * N));
                acc[0] += (double)q.x;
                acc[1] += (double)q.y;
                acc[2] += (double)q.z;
                acc[3] += (double)q.w;
            } else {
                acc[0] += (double)__builtin_nontemporal_load(p + bb * N);
            }
        }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) part[slot][c0 + v] = acc[v];
    __syncthreads();
    for (int c = t; c < TW; c += kThreads) {
        const long long j = (long long)blockIdx.x * TW + c;
        double sum = 0.0;
        for (int q = 0; q < kSlots; ++q) sum += part[q][c];
        if (j < N) out[j] = (float)sum;
    }
}

// Split reduce for narrow rows (N <= 256) over a long leading axis ("Custom
// Kernel Optimization Implementation Plan", Tasks 4-5: a batch-parallel first
// phase of block partial sums, then a final reduce of the partials; here both
// phases keep a fixed summation order).  Workgroup p sums rows
// [p R, min(B, (p+1) R)) of all N columns.  Threads t < T = (256 / N) N read
// consecutive elements (consecutive floats for consecutive threads): thread t
// owns column t % N and starts at row t / N of the chunk, stepping RP = T / N
// rows, 8 rows' loads in flight, accumulating in float64.  The RP sums of each
// column are then combined by a fixed pairwise tree through LDS, and thread
// j < N writes the chunk's sum of column j.  This is phase 1: it reads the
// float32 input and writes float64 partials [P][N]; reduce_partials_kernel is
// phase 2.
template <typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void reduce_rows_narrow_kernel(const TIn* __restrict__ in, long long B,
                                                                      int N, long long R,
                                                                      TOut* __restrict__ out) {
    __shared__ double red[kThreads];
    const int t = threadIdx.x;
    const int RP = kThreads / N, T = RP * N;
    const long long r0 = (long long)blockIdx.x * R;
    const long long r1 = min(B, r0 + R);
    double acc = 0.0;
    if (t < T) {
        const TIn* p = in + t % N;
        long long r = r0 + t / N;
        for (; r + 7LL * RP < r1; r += 8LL * RP) {
            TIn q[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) q[u] = __builtin_nontemporal_load(p + (r + (long long)u * RP) * N);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += (double)q[u];
        }
        for (; r < r1; r += RP) acc += (double)__builtin_nontemporal_load(p + r * N);
    }
    red[t] = acc;
    __syncthreads();
    // slot q = t / N adds slot q + w when q is a multiple of 2w: a fixed tree
    for (int w = 1; w < RP; w *= 2) {
        if (t < T) {
            const int q = t / N;
            if (q % (2 * w) == 0 && q + w < RP) red[t] += red[t + w * N];
        }
        __syncthreads();
    }
    if (t < N) out[(long long)blockIdx.x * N + t] = (TOut)red[t];
}

// Second phase of the split reduce: the P float64 partial rows [P][N] summed
// per column.  A workgroup owns 8 consecutive columns and has 32 row slots:
// thread t reads column 8g + t % 8 in rows t / 8, t / 8 + 32, ... (8 loads in
// flight), then the 32 slot sums of each column are combined by a fixed
// pairwise tree through LDS.  The order depends only on (P, N).
constexpr int kPartCols = 8, kPartSlots = kThreads / kPartCols;
__global__ __launch_bounds__(kThreads) void reduce_partials_kernel(const double* __restrict__ part, long long P,
                                                                   int N, float* __restrict__ out) {
    __shared__ double red[kPartSlots][kPartCols + 1];
    const int t = threadIdx.x, c = t % kPartCols, slot = t / kPartCols;
    const int col = blockIdx.x * kPartCols + c;
    double acc = 0.0;
    if (col < N) {
        const double* p = part + col;
        long long r = slot;
        for (; r + 7LL * kPartSlots < P; r += 8LL * kPartSlots) {
            double q[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) q[u] = p[(r + (long long)u * kPartSlots) * N];
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += q[u];
        }
        for (; r < P; r += kPartSlots) acc += p[r * N];
    }
    red[slot][c] = acc;
    __syncthreads();
    for (int w = 1; w < kPartSlots; w *= 2) {
        if (slot % (2 * w) == 0 && slot + w < kPartSlots) red[slot][c] += red[slot + w][c];
        __syncthreads();
    }
    if (slot == 0 && col < N) out[col] = (float)red[0][c];
}

// ---------------------------------------------------------- host helpers
struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
inline Range span(const void* p, long long elems) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + (uintptr_t)elems * sizeof(float)};
}
inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
// No output range overlaps an input range or another output range.
inline bool outputs_disjoint(const Range* outs, int n_out, const Range* ins, int n_in) {
    for (int o = 0; o < n_out; ++o) {
        for (int i = 0; i < n_in; ++i)
            if (overlap(outs[o], ins[i])) return false;
        for (int p = o + 1; p < n_out; ++p)
            if (overlap(outs[o], outs[p])) return false;
    }
    return true;
}

// Checked a*b for non-negative operands; false on overflow of the byte count.
inline bool mul_ok(long long a, long long b, long long* r) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > (LLONG_MAX / 4) / a) return false;
    *r = a * b;
    return true;
}

int check_params(const cfc_params_t* p) {
    if (!p || !p->w_in || !p->w_rec || !p->b || !p->w_tau) return CFC_ERR_NULL;
    if (p->n_in < 1 || p->n_hid < 1) return CFC_ERR_DIM;
    if (p->n_in > kMaxIn || p->n_hid > kMaxHid) return CFC_ERR_UNSUPPORTED;
    if (p->cell != CFC_CELL_GATED && p->cell != CFC_CELL_TAU_DECAY) return CFC_ERR_UNSUPPORTED;
    return CFC_OK;
}

std::once_flag g_attr_once;
void set_kernel_attributes() {
    std::call_once(g_attr_once, [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&cfc_bwd_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&cfc_fwd_small_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&cfc_bwd_small_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&cfc_bwd_small_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&cfc_fb_small_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&cfc_fb_small_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&cfc_fwd_large_kernel<false, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&cfc_fwd_large_kernel<false, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        for (const void* f : {reinterpret_cast<const void*>(&cfc_fwd_large32_kernel<false, false>),
                              reinterpret_cast<const void*>(&cfc_fwd_large32_kernel<true, false>),
                              reinterpret_cast<const void*>(&cfc_fwd_large32_kernel<true, true>)})
            (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        for (const void* f : {reinterpret_cast<const void*>(&cfc_bwd_large_kernel<false, false, false>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, false, false>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<false, true, false>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, true, false>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<false, false, true, 1>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, false, true, 1>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<false, true, true, 1>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, true, true, 1>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<false, false, true, 2>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, false, true, 2>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<false, true, true, 2>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, true, true, 2>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<false, false, false, 0, true>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, false, false, 0, true>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<false, true, false, 0, true>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, true, false, 0, true>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, false, true, 1, true>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, true, true, 1, true>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, false, false, 1, true>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_kernel<true, true, false, 1, true>)})
            (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        for (const void* f : {reinterpret_cast<const void*>(&cfc_bwd_large_grads_kernel<false>),
                              reinterpret_cast<const void*>(&cfc_bwd_large_grads_kernel<true>)})
            (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGradsLdsReserve);
    });
}

// The 16-row kernels' unmasked instance: exact 256 x 256 shapes, 16-byte aligned weights.
inline bool large_full(const cfc_params_t* p) {
    return p->n_in == kLarge && p->n_hid == kLarge && (reinterpret_cast<uintptr_t>(p->w_in) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(p->w_rec) & 15) == 0;
}

inline int launch_status() { return hipGetLastError() == hipSuccess ? CFC_OK : CFC_ERR_HIP; }

}  // namespace

// ================================================================ C ABI
extern "C" long long cfc_scratch_row_len(int n_in, int n_hid) {
    if (n_in < 1 || n_hid < 1) return -1;
    const long long w = (long long)n_in + (long long)n_hid + 2;
    long long n;
    if (!mul_ok(w, n_hid, &n)) return -1;
    return n;
}

extern "C" const char* cfc_status_string(int code) {
    switch (code) {
        case CFC_OK: return "ok";
        case CFC_ERR_NULL: return "null pointer argument";
        case CFC_ERR_DIM: return "dimension out of range or size overflow";
        case CFC_ERR_DT: return "dt is not finite";
        case CFC_ERR_UNSUPPORTED: return "shape beyond the compiled kernel limits";
        case CFC_ERR_OVERLAP: return "output range overlaps another argument";
        case CFC_ERR_HIP: return "HIP launch error";
        default: return "unknown status code";
    }
}

extern "C" int cfc_forward(const cfc_params_t* params, const float* x, const float* h0, float dt,
                           int B, int K, float* h_seq, hipStream_t stream) {
    int rc = check_params(params);
    if (rc) return rc;
    if (!x || !h0 || !h_seq) return CFC_ERR_NULL;
    if (B < 1 || K < 1) return CFC_ERR_DIM;
    if (!std::isfinite(dt)) return CFC_ERR_DT;
    const int n_in = params->n_in, H = params->n_hid;
    long long nx, ns;
    if (!mul_ok((long long)B * K, n_in, &nx) || !mul_ok((long long)B * K, H, &ns)) return CFC_ERR_DIM;
    const Range out = span(h_seq, ns);
    const Range ins[] = {span(x, nx), span(h0, (long long)B * H), span(params->w_in, (long long)H * n_in),
                         span(params->w_rec, (long long)H * H), span(params->b, H), span(params->w_tau, H)};
    for (const Range& r : ins)
        if (overlap(out, r)) return CFC_ERR_OVERLAP;

    set_kernel_attributes();
    if (n_in <= kSmall && H <= kSmall) {
        hipLaunchKernelGGL(cfc_fwd_small_kernel, dim3(B), dim3(kThreads), small_fwd_lds_bytes(), stream,
                           params->w_in, params->w_rec, params->b, params->w_tau, x, h0, (double)dt, K,
                           n_in, H, h_seq, params->cell);
        return launch_status();
    }
    if (large_full(params)) {
        const long long groups = ((long long)B + kLR2 - 1) / kLR2;
        hipLaunchKernelGGL((cfc_fwd_large32_kernel<false, false>), dim3((unsigned)groups), dim3(kThreads),
                           large32_fwd_lds_bytes(), stream, params->w_in, params->w_rec, params->b, params->w_tau, x,
                           h0, (double)dt, B, K, h_seq, params->cell, nullptr, 0LL, nullptr, 0LL);
        return launch_status();
    }
    const long long groups = ((long long)B + kLR - 1) / kLR;
    hipLaunchKernelGGL((cfc_fwd_large_kernel<false, false>), dim3((unsigned)groups), dim3(kThreads),
                       large_fwd_lds_bytes(), stream, params->w_in, params->w_rec, params->b, params->w_tau, x, h0,
                       (double)dt, B, K, n_in, H, h_seq, params->cell, nullptr, 0LL);
    return launch_status();
}

extern "C" long long cfc_backward_workspace(int B, int Kw, int n_in, int n_hid, int flags) {
    if (B < 1 || Kw < 1 || n_in < 1 || n_hid < 1) return -1;
    if (flags != CFC_OVERWRITE && flags != CFC_ACCUMULATE) return -1;
    if (cfc_scratch_row_len(n_in, n_hid) < 0) return -1;
    const bool wide = n_in > kSmall || n_hid > kSmall;
    if (!wide || Kw > kLargeBwdMaxK || flags != CFC_ACCUMULATE) return 0;
    long long n;  // dL/da of every row-step in float64
    if (!mul_ok(8LL * B * Kw, n_hid, &n)) return -1;
    return n;
}

extern "C" long long cfc_forward_backward_workspace(int B, int K, int n_in, int n_hid, int flags) {
    const long long n = cfc_backward_workspace(B, K, n_in, n_hid, flags);
    if (n <= 0) return n;
    // accumulate mode at 256 x 256 with K <= 8: the forward's float64 weight
    // copy after the parked values
    if (n_in == kLarge && n_hid == kLarge && K <= kGradsMaxK)
        return n <= LLONG_MAX - kWideElems * 8 ? n + kWideElems * 8 : -1;
    return n;
}

namespace {
// Validation and dispatch shared by cfc_backward (one window covering all K
// steps, seeded from y), cfc_backward_window and cfc_backward_window_ws.
int backward_window(const cfc_params_t* params, const float* x, const float* h0, const float* h_seq,
                    const float* y, const float* delta_in, float dt, int B, int K, int k_begin, int k_end,
                    float* scratch, float* loss, float* grad_x, float* delta_out, int flags, void* workspace,
                    long long workspace_bytes, hipStream_t stream) {
    int rc = check_params(params);
    if (rc) return rc;
    if (!x || !h0 || !h_seq || !scratch) return CFC_ERR_NULL;
    if (!delta_in && !y) return CFC_ERR_NULL;
    if (B < 1 || K < 1 || k_begin < 0 || k_end > K || k_begin >= k_end) return CFC_ERR_DIM;
    if (!delta_in && k_end != K) return CFC_ERR_DIM;  // the loss seed belongs to the last step
    if (delta_in && loss) return CFC_ERR_DIM;          // the loss is the seeded window's
    if (flags != CFC_OVERWRITE && flags != CFC_ACCUMULATE) return CFC_ERR_DIM;
    if (!std::isfinite(dt)) return CFC_ERR_DT;
    const int n_in = params->n_in, H = params->n_hid;
    const int Kw = k_end - k_begin;
    const long long N = cfc_scratch_row_len(n_in, H);
    long long nx, ns, nsc;
    if (N < 0 || !mul_ok((long long)B * K, n_in, &nx) || !mul_ok((long long)B * K, H, &ns) ||
        !mul_ok((long long)B, N, &nsc))
        return CFC_ERR_DIM;
    // accumulate mode in the 16-row kernel parks dL/da in the workspace
    const long long ws_need = cfc_backward_workspace(B, Kw, n_in, H, flags);
    if (ws_need < 0) return CFC_ERR_DIM;
    if (workspace && ws_need > 0 &&
        (workspace_bytes < ws_need || (reinterpret_cast<uintptr_t>(workspace) & 7) != 0))
        return CFC_ERR_DIM;
    const bool ws_used = workspace && ws_need > 0;
    const bool small = n_in <= kSmall && H <= kSmall && Kw <= kSmallBwdMaxK;
    const bool large = !small && (n_in > kSmall || H > kSmall) && Kw <= kLargeBwdMaxK &&
                       (flags == CFC_OVERWRITE || ws_used);
    const size_t lds = small ? small_bwd_lds_bytes() : large ? large_bwd_lds_bytes() : bwd_lds_bytes(Kw, n_in, H);
    if (lds > kLdsBytes) return CFC_ERR_UNSUPPORTED;
    const long long BH = (long long)B * H;
    const Range outs[] = {span(scratch, nsc), span(loss, loss ? B : 0), span(grad_x, grad_x ? nx : 0),
                          span(delta_out, delta_out && delta_out != delta_in ? BH : 0),
                          Range{reinterpret_cast<uintptr_t>(workspace),
                                reinterpret_cast<uintptr_t>(workspace) + (ws_used ? (uintptr_t)ws_need : 0)}};
    const Range ins[] = {span(x, nx), span(h0, BH), span(h_seq, ns), span(y, y && !delta_in ? BH : 0),
                         span(delta_in, delta_in ? BH : 0), span(params->w_in, (long long)H * n_in),
                         span(params->w_rec, (long long)H * H), span(params->b, H), span(params->w_tau, H)};
    if (!outputs_disjoint(outs, 5, ins, 9)) return CFC_ERR_OVERLAP;
    if (delta_out && delta_out == delta_in) {  // in place: still disjoint from the other outputs
        const Range d = span(delta_out, BH);
        for (int o : {0, 1, 2, 4})
            if (overlap(d, outs[o])) return CFC_ERR_OVERLAP;
    }
    const BwdWindow win{K, k_begin, Kw, delta_in, delta_out};
    set_kernel_attributes();
    if (small) {
        auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
        const bool whole = Kw == kSmallBwdMaxK && n_in == kSmall && H == kSmall && al16(x) && al16(h0) &&
                           al16(h_seq) && al16(params->w_in) && al16(params->w_rec);
        auto kern = whole ? &cfc_bwd_small_kernel<true> : &cfc_bwd_small_kernel<false>;
        hipLaunchKernelGGL(kern, dim3(B), dim3(kThreads), lds, stream, params->w_in,
                           params->w_rec, params->b, params->w_tau, x, h0, h_seq, y, (double)dt, win, n_in, H,
                           scratch, loss, grad_x, flags == CFC_ACCUMULATE ? 1 : 0, params->cell);
        return launch_status();
    }
    if (large) {
        const long long groups = ((long long)B + kLR - 1) / kLR;
        const bool tau = params->cell == CFC_CELL_TAU_DECAY, full = large_full(params);
        auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
        // accumulating a whole sequence at exactly 256 x 256, K <= 8: phase 1
        // alone (dL/da into the workspace, dL/dw_tau added to the scratch),
        // then the vector phase 2's read-add-write
        if (full && flags == CFC_ACCUMULATE && k_begin == 0 && Kw == K && !delta_in && K <= kGradsMaxK &&
            al16(x) && al16(h0) && al16(h_seq) && al16(scratch)) {
            auto st1 = tau ? &cfc_bwd_large_kernel<true, true, false, 1, true>
                           : &cfc_bwd_large_kernel<true, false, false, 1, true>;
            hipLaunchKernelGGL(st1, dim3((unsigned)groups), dim3(kThreads), lds, stream, params->w_in, params->w_rec,
                               params->b, params->w_tau, x, h0, h_seq, y, (double)dt, B, win, n_in, H, scratch, loss,
                               grad_x, static_cast<unsigned*>(workspace), nullptr, 0LL);
            const int rc = launch_status();
            if (rc) return rc;
            hipLaunchKernelGGL(cfc_bwd_large_grads_kernel<true>, dim3((unsigned)B), dim3(kThreads), kGradsLdsReserve,
                               stream, x, h0, h_seq, K, scratch, N, static_cast<const unsigned*>(workspace));
            return launch_status();
        }
        auto kern = full ? (tau ? &cfc_bwd_large_kernel<true, true, false> : &cfc_bwd_large_kernel<true, false, false>)
                         : (tau ? &cfc_bwd_large_kernel<false, true, false> : &cfc_bwd_large_kernel<false, false, false>);
        if (flags == CFC_ACCUMULATE)
            kern = full ? (tau ? &cfc_bwd_large_kernel<true, true, false, 0, true>
                               : &cfc_bwd_large_kernel<true, false, false, 0, true>)
                        : (tau ? &cfc_bwd_large_kernel<false, true, false, 0, true>
                               : &cfc_bwd_large_kernel<false, false, false, 0, true>);
        hipLaunchKernelGGL(kern, dim3((unsigned)groups), dim3(kThreads), lds, stream, params->w_in, params->w_rec,
                           params->b, params->w_tau, x, h0, h_seq, y, (double)dt, B, win, n_in, H, scratch, loss,
                           grad_x, ws_used ? static_cast<unsigned*>(workspace) : nullptr, nullptr, 0LL);
        return launch_status();
    }
    hipLaunchKernelGGL(cfc_bwd_kernel, dim3(B), dim3(kThreads), lds, stream, params->w_in,
                       params->w_rec, params->b, params->w_tau, x, h0, h_seq, y, (double)dt, win, n_in,
                       H, scratch, loss, grad_x, flags == CFC_ACCUMULATE ? 1 : 0, params->cell);
    return launch_status();
}
}  // namespace

extern "C" int cfc_backward(const cfc_params_t* params, const float* x, const float* h0,
                            const float* h_seq, const float* y, float dt, int B, int K,
                            float* scratch, float* loss, float* grad_x, float* grad_h0, int flags,
                            hipStream_t stream) {
    if (!y) return CFC_ERR_NULL;
    return backward_window(params, x, h0, h_seq, y, nullptr, dt, B, K, 0, K, scratch, loss, grad_x, grad_h0,
                           flags, nullptr, 0, stream);
}

extern "C" int cfc_backward_window(const cfc_params_t* params, const float* x, const float* h0,
                                   const float* h_seq, const float* y, const float* delta_in, float dt,
                                   int B, int K, int k_begin, int k_end, float* scratch, float* loss,
                                   float* grad_x, float* delta_out, int flags, hipStream_t stream) {
    return backward_window(params, x, h0, h_seq, y, delta_in, dt, B, K, k_begin, k_end, scratch, loss, grad_x,
                           delta_out, flags, nullptr, 0, stream);
}

extern "C" int cfc_backward_window_ws(const cfc_params_t* params, const float* x, const float* h0,
                                      const float* h_seq, const float* y, const float* delta_in, float dt,
                                      int B, int K, int k_begin, int k_end, float* scratch, float* loss,
                                      float* grad_x, float* delta_out, int flags, void* workspace,
                                      long long workspace_bytes, hipStream_t stream) {
    return backward_window(params, x, h0, h_seq, y, delta_in, dt, B, K, k_begin, k_end, scratch, loss, grad_x,
                           delta_out, flags, workspace, workspace_bytes, stream);
}

namespace {
int forward_backward(const cfc_params_t* params, const float* x, const float* h0, const float* y, float dt, int B,
                     int K, float* h_seq, float* scratch, float* loss, float* grad_x, float* grad_h0, int flags,
                     void* workspace, long long workspace_bytes, hipStream_t stream) {
    int rc = check_params(params);
    if (rc) return rc;
    if (!x || !h0 || !y || !h_seq || !scratch) return CFC_ERR_NULL;
    if (B < 1 || K < 1) return CFC_ERR_DIM;
    if (flags != CFC_OVERWRITE && flags != CFC_ACCUMULATE) return CFC_ERR_DIM;
    if (!std::isfinite(dt)) return CFC_ERR_DT;
    const int n_in = params->n_in, H = params->n_hid;
    const long long N = cfc_scratch_row_len(n_in, H);
    long long nx, ns, nsc;
    if (N < 0 || !mul_ok((long long)B * K, n_in, &nx) || !mul_ok((long long)B * K, H, &ns) ||
        !mul_ok((long long)B, N, &nsc))
        return CFC_ERR_DIM;
    const Range outs[] = {span(h_seq, ns), span(scratch, nsc), span(loss, loss ? B : 0),
                          span(grad_x, grad_x ? nx : 0), span(grad_h0, grad_h0 ? (long long)B * H : 0)};
    const Range ins[] = {span(x, nx), span(h0, (long long)B * H), span(y, (long long)B * H),
                         span(params->w_in, (long long)H * n_in), span(params->w_rec, (long long)H * H),
                         span(params->b, H), span(params->w_tau, H)};
    if (!outputs_disjoint(outs, 5, ins, 7)) return CFC_ERR_OVERLAP;
    if (n_in <= kSmall && H <= kSmall && K <= kSmallBwdMaxK) {
        set_kernel_attributes();
        // the whole-shape instance reads x, W_in and W_rec as float4 without checks
        auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
        const bool whole = K == kSmallBwdMaxK && n_in == kSmall && H == kSmall && al16(params->w_in) &&
                           al16(params->w_rec) && al16(x);
        auto* kern = whole ? &cfc_fb_small_kernel<true> : &cfc_fb_small_kernel<false>;
        hipLaunchKernelGGL(kern, dim3(B), dim3(kThreads), small_fb_lds_bytes(), stream,
                           params->w_in, params->w_rec, params->b, params->w_tau, x, h0, y, (double)dt, K,
                           n_in, H, h_seq, scratch, loss, grad_x, grad_h0, flags == CFC_ACCUMULATE ? 1 : 0,
                           params->cell);
        return launch_status();
    }
    // other shapes: the two directions as separate launches on the same stream;
    // the backward's shape limits and workspace are checked before anything is
    // launched
    const long long ws_need = cfc_backward_workspace(B, K, n_in, H, flags);
    if (ws_need < 0) return CFC_ERR_DIM;
    const bool ws_used = workspace && ws_need > 0;
    // a workspace of cfc_forward_backward_workspace bytes also holds the
    // float64 weight copy of the accumulate path at 256 x 256
    const long long ws_full = cfc_forward_backward_workspace(B, K, n_in, H, flags);
    const bool ws_wide = ws_used && ws_full > ws_need && workspace_bytes >= ws_full;
    if (ws_used) {
        if (workspace_bytes < ws_need || (reinterpret_cast<uintptr_t>(workspace) & 7) != 0) return CFC_ERR_DIM;
        const Range w{reinterpret_cast<uintptr_t>(workspace),
                      reinterpret_cast<uintptr_t>(workspace) + (uintptr_t)(ws_wide ? ws_full : ws_need)};
        if (!outputs_disjoint(&w, 1, outs, 5) || !outputs_disjoint(&w, 1, ins, 7)) return CFC_ERR_OVERLAP;
    }
    const bool large = (n_in > kSmall || H > kSmall) && K <= kLargeBwdMaxK && (flags == CFC_OVERWRITE || ws_used);
    const bool small_bwd = n_in <= kSmall && H <= kSmall && K <= kSmallBwdMaxK;
    const size_t lds = small_bwd ? small_bwd_lds_bytes() : large ? large_bwd_lds_bytes() : bwd_lds_bytes(K, n_in, H);
    if (lds > kLdsBytes) return CFC_ERR_UNSUPPORTED;
    const auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    // accumulate mode at exactly 256 x 256 and K <= 8 with a workspace: the
    // forward parks a_k in the workspace (rows of 2 K H words), the parked
    // phase 1 turns it into dL/da there and adds dL/dw_tau into the scratch,
    // and the vector phase 2 adds the weight gradients and db
    if (large && flags == CFC_ACCUMULATE && ws_used && large_full(params) && K <= kGradsMaxK && al16(x) &&
        al16(h0) && al16(h_seq) && al16(scratch)) {
        set_kernel_attributes();
        const bool tau = params->cell == CFC_CELL_TAU_DECAY;
        // the float64 weight copy after the parks, where the workspace has
        // room for it (cfc_forward_backward_workspace) and is 16-byte aligned
        float* wide = nullptr;
        if (ws_wide && al16(workspace)) {
            wide = reinterpret_cast<float*>(workspace) + 2LL * B * K * H;
            hipLaunchKernelGGL(widen_weights_kernel, dim3((unsigned)(kWideElems / kThreads)), dim3(kThreads), 0,
                               stream, params->w_in, params->w_rec, wide, kWideQuarterFloats);
        }
        auto fwd = wide ? &cfc_fwd_large32_kernel<true, true> : &cfc_fwd_large32_kernel<true, false>;
        hipLaunchKernelGGL(fwd, dim3((unsigned)(((long long)B + kLR2 - 1) / kLR2)), dim3(kThreads),
                           large32_fwd_lds_bytes(), stream, params->w_in, params->w_rec, params->b, params->w_tau, x, h0,
                           (double)dt, B, K, h_seq, params->cell, reinterpret_cast<float*>(workspace), 2LL * K * H,
                           wide, kWideQuarterFloats);
        rc = launch_status();
        if (rc) return rc;
        const BwdWindow win{K, 0, K, nullptr, grad_h0};
        auto bwd1 = tau ? &cfc_bwd_large_kernel<true, true, true, 1, true> : &cfc_bwd_large_kernel<true, false, true, 1, true>;
        hipLaunchKernelGGL(bwd1, dim3((unsigned)(((long long)B + kLR - 1) / kLR)), dim3(kThreads), large_bwd_lds_bytes(),
                           stream, params->w_in, params->w_rec, params->b, params->w_tau, x, h0, h_seq, y, (double)dt,
                           B, win, n_in, H, scratch, loss, grad_x, static_cast<unsigned*>(workspace), wide,
                           kWideQuarterFloats);
        rc = launch_status();
        if (rc) return rc;
        hipLaunchKernelGGL(cfc_bwd_large_grads_kernel<true>, dim3((unsigned)B), dim3(kThreads), kGradsLdsReserve, stream,
                           x, h0, h_seq, K, scratch, N, static_cast<const unsigned*>(workspace));
        return launch_status();
    }
    // 16-row kernels in overwrite mode: the forward parks a_k (float64) in the
    // head [0, 2KH) of each scratch row and the backward reads it back instead
    // of recomputing it, parking dL/da_k over a_k (needs 8-byte-aligned rows;
    // the head and the dL/dw_tau sums in [N - 2H, N) are disjoint, and so is
    // the widened weight copy between them, because 4KH <= N here)
    if (large && flags == CFC_OVERWRITE && N % 2 == 0 && (reinterpret_cast<uintptr_t>(scratch) & 7) == 0 &&
        4LL * K * H <= N) {
        set_kernel_attributes();
        const long long groups = ((long long)B + kLR - 1) / kLR;
        const bool full = large_full(params), tau = params->cell == CFC_CELL_TAU_DECAY;
        // float64 weights for the 256 x 256 products, in the middle of
        // scratch rows 0..3 (16-byte aligned for their double2 loads)
        const bool use_wide = full && B >= 4 && al16(scratch) && N % 4 == 0 && 4LL * K * H + kWideElems / 2 <= N;
        float* wide = use_wide ? scratch + 2LL * K * H : nullptr;
        if (use_wide) {
            hipLaunchKernelGGL(widen_weights_kernel, dim3((unsigned)(kWideElems / kThreads)), dim3(kThreads), 0,
                               stream, params->w_in, params->w_rec, wide, N);
            hipLaunchKernelGGL((cfc_fwd_large32_kernel<true, true>), dim3((unsigned)(((long long)B + kLR2 - 1) / kLR2)),
                               dim3(kThreads), large32_fwd_lds_bytes(), stream, params->w_in, params->w_rec, params->b,
                               params->w_tau, x, h0, (double)dt, B, K, h_seq, params->cell, scratch, N, wide, N);
        } else if (full) {
            hipLaunchKernelGGL((cfc_fwd_large32_kernel<true, false>), dim3((unsigned)(((long long)B + kLR2 - 1) / kLR2)),
                               dim3(kThreads), large32_fwd_lds_bytes(), stream, params->w_in, params->w_rec, params->b,
                               params->w_tau, x, h0, (double)dt, B, K, h_seq, params->cell, scratch, N, nullptr, 0LL);
        } else
            hipLaunchKernelGGL((cfc_fwd_large_kernel<false, true>), dim3((unsigned)groups), dim3(kThreads),
                               large_fwd_lds_bytes(), stream, params->w_in, params->w_rec, params->b, params->w_tau, x,
                               h0, (double)dt, B, K, n_in, H, h_seq, params->cell, scratch, N);
        rc = launch_status();
        if (rc) return rc;
        auto bwd1 = full ? (tau ? &cfc_bwd_large_kernel<true, true, true, 1> : &cfc_bwd_large_kernel<true, false, true, 1>)
                         : (tau ? &cfc_bwd_large_kernel<false, true, true, 1> : &cfc_bwd_large_kernel<false, false, true, 1>);
        auto bwd2 = full ? (tau ? &cfc_bwd_large_kernel<true, true, true, 2> : &cfc_bwd_large_kernel<true, false, true, 2>)
                         : (tau ? &cfc_bwd_large_kernel<false, true, true, 2> : &cfc_bwd_large_kernel<false, false, true, 2>);
        const BwdWindow win{K, 0, K, nullptr, grad_h0};
        // phase 2 on the vector units where it applies (256 x 256, K <= 8,
        // x, h0, h_seq and the scratch 16-byte aligned for its float4 accesses)
        const bool vgrads = full && K <= kGradsMaxK && al16(x) && al16(h0) && al16(h_seq) && al16(scratch);
        for (auto* bwd : {bwd1, bwd2}) {
            if (vgrads && bwd == bwd2) {
                hipLaunchKernelGGL(cfc_bwd_large_grads_kernel<false>, dim3((unsigned)B), dim3(kThreads), kGradsLdsReserve,
                                   stream, x, h0, h_seq, K, scratch, N, nullptr);
                break;
            }
            hipLaunchKernelGGL(bwd, dim3((unsigned)groups), dim3(kThreads), large_bwd_lds_bytes(), stream, params->w_in,
                               params->w_rec, params->b, params->w_tau, x, h0, h_seq, y, (double)dt, B, win, n_in, H,
                               scratch, loss, grad_x, nullptr, bwd == bwd1 ? wide : nullptr, N);
        }
        return launch_status();
    }
    rc = cfc_forward(params, x, h0, dt, B, K, h_seq, stream);
    if (rc) return rc;
    return backward_window(params, x, h0, h_seq, y, nullptr, dt, B, K, 0, K, scratch, loss, grad_x, grad_h0, flags,
                           workspace, workspace_bytes, stream);
}
}  // namespace

extern "C" int cfc_forward_backward(const cfc_params_t* params, const float* x, const float* h0,
                                    const float* y, float dt, int B, int K, float* h_seq, float* scratch,
                                    float* loss, float* grad_x, float* grad_h0, int flags,
                                    hipStream_t stream) {
    return forward_backward(params, x, h0, y, dt, B, K, h_seq, scratch, loss, grad_x, grad_h0, flags, nullptr, 0,
                            stream);
}

extern "C" int cfc_forward_backward_ws(const cfc_params_t* params, const float* x, const float* h0,
                                       const float* y, float dt, int B, int K, float* h_seq, float* scratch,
                                       float* loss, float* grad_x, float* grad_h0, int flags, void* workspace,
                                       long long workspace_bytes, hipStream_t stream) {
    return forward_backward(params, x, h0, y, dt, B, K, h_seq, scratch, loss, grad_x, grad_h0, flags, workspace,
                            workspace_bytes, stream);
}

// Chunking of the split reduce; it depends only on (B, N), so the summation
// order -- and the result -- is the same on every device.  At most 1024
// chunks and 256 K partials (2 MB of workspace); each chunk is at least 8
// passes of RP rows.
constexpr long long kSplitMaxChunks = 1024;
constexpr long long kSplitMaxPartials = 262144;
struct SplitPlan {
    long long R, P;
};
inline SplitPlan split_plan(long long B, long long N) {
    const long long RP = kThreads / N;
    const long long chunks = std::min(kSplitMaxChunks, kSplitMaxPartials / N);
    long long R = std::max((B + chunks - 1) / chunks, 8 * RP);
    R = (R + RP - 1) / RP * RP;
    return SplitPlan{R, B > 0 ? (B + R - 1) / R : 0};
}

extern "C" long long reduce_axis0_split_workspace(long long B, long long N) {
    if (B < 0 || N < 0) return -1;
    long long n;
    if (!mul_ok(B, N, &n)) return -1;
    if (N == 0 || N > kThreads) return 0;
    const SplitPlan sp = split_plan(B, N);
    return sp.P >= 2 ? sp.P * N * (long long)sizeof(double) : 0;
}

extern "C" int reduce_axis0_split(const float* per_batch, long long B, long long N, float* out,
                                  void* workspace, long long workspace_bytes, hipStream_t stream) {
    const long long need = reduce_axis0_split_workspace(B, N);
    if (need < 0) return CFC_ERR_DIM;
    if (need == 0) return reduce_axis0(per_batch, B, N, out, stream);
    if (!out || !per_batch || !workspace) return CFC_ERR_NULL;
    if (workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7) != 0) return CFC_ERR_DIM;
    const Range ws{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + (uintptr_t)need};
    const Range in = span(per_batch, B * N), o = span(out, N);
    if (overlap(o, in) || overlap(ws, in) || overlap(ws, o)) return CFC_ERR_OVERLAP;
    const SplitPlan sp = split_plan(B, N);
    double* part = static_cast<double*>(workspace);
    hipLaunchKernelGGL((reduce_rows_narrow_kernel<float, double>), dim3((unsigned)sp.P), dim3(kThreads), 0, stream,
                       per_batch, B, (int)N, sp.R, part);
    hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)((N + kPartCols - 1) / kPartCols)), dim3(kThreads), 0,
                       stream, (const double*)part, sp.P, (int)N, out);
    return launch_status();
}

// The allocation-free variant's partials: one static array per GPU (each
// device holds its own copy at its own address).  In host code `scratch` is
// only a handle for hipGetSymbolAddress; kernels get the per-device address
// resolved below.
static_assert(CFC_SPLIT_STATIC_BYTES == kSplitMaxPartials * (long long)sizeof(double),
              "the static array holds the largest split plan's partials");
static __device__ __align__(256) double scratch[kSplitMaxPartials];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, resolved once per
// device with that device current; nullptr on failure.
void* static_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int reduce_axis0_split_noalloc(const float* per_batch, long long B, long long N, float* out,
                                          hipStream_t stream) {
    const long long need = reduce_axis0_split_workspace(B, N);
    if (need < 0) return CFC_ERR_DIM;
    if (need == 0) return reduce_axis0(per_batch, B, N, out, stream);
    if (!out || !per_batch) return CFC_ERR_NULL;
    if (need > CFC_SPLIT_STATIC_BYTES) return CFC_ERR_UNSUPPORTED;
    if (overlap(span(out, N), span(per_batch, B * N))) return CFC_ERR_OVERLAP;
    void* ws = static_scratch();
    if (!ws) return CFC_ERR_HIP;
    const SplitPlan sp = split_plan(B, N);
    double* part = static_cast<double*>(ws);
    hipLaunchKernelGGL((reduce_rows_narrow_kernel<float, double>), dim3((unsigned)sp.P), dim3(kThreads), 0, stream,
                       per_batch, B, (int)N, sp.R, part);
    hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)((N + kPartCols - 1) / kPartCols)), dim3(kThreads), 0,
                       stream, (const double*)part, sp.P, (int)N, out);
    return launch_status();
}

extern "C" int reduce_axis0(const float* per_batch, long long B, long long N, float* out,
                            hipStream_t stream) {
    if (B < 0 || N < 0) return CFC_ERR_DIM;
    long long n;
    if (!mul_ok(B, N, &n)) return CFC_ERR_DIM;
    if (N == 0) return CFC_OK;
    if (!out || (B > 0 && !per_batch)) return CFC_ERR_NULL;
    if (B > 0 && overlap(span(out, N), span(per_batch, n))) return CFC_ERR_OVERLAP;
    const bool vec4 = (N % 4 == 0) && (reinterpret_cast<uintptr_t>(per_batch) % 16 == 0);
    // 256-byte row segments (16 lanes x float4, 8 rows' loads in flight per
    // slot); above 256 MB of input (more than the MALL holds), 512-byte
    // segments with 16 rows in flight: measured on MI355X at [8192, 131584]
    // 0.696 against 0.711 ms after the large-batch backward, while at the
    // training-scale scratch (34 MB) they were 0.5 us slower.  The two
    // group the rows differently, so the result depends on (B, N) only.
    const bool wide_tiles = vec4 && n > (64LL << 20);  // n floats: more than 256 MB
    const long long tw = wide_tiles ? 128 : 64;
    const long long tiles = (N + tw - 1) / tw;
    if (tiles > INT_MAX) return CFC_ERR_DIM;
    if (wide_tiles)
        hipLaunchKernelGGL((reduce_axis0_kernel<4, 32>), dim3((unsigned)tiles), dim3(kThreads), 0, stream,
                           per_batch, B, N, out);
    else if (vec4)
        hipLaunchKernelGGL((reduce_axis0_kernel<4, 16>), dim3((unsigned)tiles), dim3(kThreads), 0, stream,
                           per_batch, B, N, out);
    else
        hipLaunchKernelGGL((reduce_axis0_kernel<1, 64>), dim3((unsigned)tiles), dim3(kThreads), 0, stream,
                           per_batch, B, N, out);
    return launch_status();
}

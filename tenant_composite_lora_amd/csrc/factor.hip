// Retained-rank producer (LoRAForge, approach (2) and approach (3); Figure 3
// for the schedule of the batched QR).
//
// A module's LoRA update is Delta W = X Y with X = B (d_out x r, tall and
// skinny; its columns are the rows of B_t) and Y = A^T (the rows of A_t).
// The balanced factors come from four launches over a batch of modules of
// one shape:
//   1. tsqr_leaf    one wave per (module, row tile of X): Householder QR of
//                   the tile, 512 - RT (rank <= 16) or 256 - RT new rows at a
//                   time stacked under the running R, in registers (lane i
//                   holds rows i, 64 + i, ...).
//                   Writes the tile's R.
//   2. gram_kernel  one wave per (module, column slice of Y): the slice's
//                   share of G = Y Y^T on the matrix cores (bf16 in, fp32
//                   accumulation).
//   3. factor_core  one wave per module: merges the tiles' R factors
//                   (the same Householder pass over two stacked R), then, in
//                   fp64, H H^T = R G R^T (H = R Y is never formed), a
//                   parallel cyclic Jacobi eigensolver, the spectrum sorted
//                   largest first, and the two r x r maps
//                     Mt = S^(-1/2) U^T R        (T = Mt Y)
//                     Mf = S^(-3/2) U^T R G      (F^T = Mf X^T)
//                   F = X Y T^T S^(-1), so Q is applied implicitly and never
//                   stored; no triangular solve, so a rank-deficient X needs
//                   no special case.
//   4. factor_out   F^T and T, bf16, one pass over B_t and A_t.
// Directions with eigenvalue at most 2^-23 of the largest (the rounding
// level of the fp32 Gram) are taken as exactly zero: sigma 0, zero rows.
#include <algorithm>
#include <cmath>
#include <vector>

#include "tcl_internal.hpp"

namespace tcl {
namespace {

constexpr int kFacWaves = 4;      // waves per workgroup of the leaf and Gram kernels
constexpr int kFacMaxRank = 32;   // largest rank built
constexpr int kLeafWaveTarget = 8192;
constexpr int kGramWaveTarget = 4096;
constexpr int kMaxLeaves = 64;
constexpr int kJacobiSweeps = 16;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 fbf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float ff32x4_t;

struct FacArgs {
  const uint16_t *Bt, *At;  // [M][r][d_out], [M][r][d_in], bf16 bits
  uint16_t *Ft, *T;         // same layouts
  float *sigma;             // [M][r]
  float *leafR;             // [M][P][RT][RT]
  float *gpart;             // [M][S][RT][RT]
  float *mats;              // [M][2][RT][RT]: Mf, then Mt
  int M, d_out, d_in, r, P, S, rows_per_leaf, cols_per_split;
};

__device__ inline uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return uint16_t((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Sum over the 64 lanes with DPP moves: shifts of 1, 2, 4, 8 lanes inside
// each row of 16, then the row broadcasts; lane 63 holds the total, which is
// read as a uniform value.  Fixed order, so the same on every run.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

__device__ inline float wave_total(float v) {
  v = dpp_add<0x111, 0xf>(v);
  v = dpp_add<0x112, 0xf>(v);
  v = dpp_add<0x114, 0xf>(v);
  v = dpp_add<0x118, 0xf>(v);
  v = dpp_add<0x142, 0xa>(v);
  v = dpp_add<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ inline float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Householder QR of the 64 * RPL rows one wave holds (row 64 s + lane in
// x[s]; RT columns).  Afterwards rows 0..RT-1 (x[0] of lanes 0..RT-1) hold
// the upper triangular R of the rows' span (up to row signs) and every row
// below is zero.  Column j's reflector is v = x_j - beta e_j over rows >= j
// with beta = -sign(alpha) |x_j|; v^T x_c is read off the Gram row
// g_c = sum_{rows >= j} x_j x_c as g_c - beta x[j][c], so each column costs
// one batch of wave sums whatever the number of rows.
template <int RT, int RPL>
__device__ inline void hh_pass(float (&x)[RPL][RT], int lane) {
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    float g[RT];
#pragma unroll
    for (int c = j; c < RT; ++c) {
      float p = lane >= j ? x[0][j] * x[0][c] : 0.f;
#pragma unroll
      for (int sl = 1; sl < RPL; ++sl) p += x[sl][j] * x[sl][c];
      g[c] = wave_total(p);
    }
    const float nrm2 = g[j];
    if (nrm2 > 1e-30f) {  // below this the column is zero to fp32 precision
      const float alpha = lane_value(x[0][j], j);
      const float beta = alpha >= 0.f ? -sqrtf(nrm2) : sqrtf(nrm2);
      const float f = 1.f / (beta * (beta - alpha));
      float v[RPL];
      v[0] = lane > j ? x[0][j] : (lane == j ? alpha - beta : 0.f);
#pragma unroll
      for (int sl = 1; sl < RPL; ++sl) v[sl] = x[sl][j];
#pragma unroll
      for (int c = j + 1; c < RT; ++c) {
        const float w = f * (g[c] - beta * lane_value(x[0][c], j));
#pragma unroll
        for (int sl = 0; sl < RPL; ++sl) x[sl][c] -= v[sl] * w;
      }
      x[0][j] = lane == j ? beta : (lane > j ? 0.f : x[0][j]);
#pragma unroll
      for (int sl = 1; sl < RPL; ++sl) x[sl][j] = 0.f;
    }
  }
}

// Rows per lane of the leaf pass: 512 rows per wave at rank 16, 256 at 32.
template <int RT>
constexpr int leaf_rpl() { return RT <= 16 ? 8 : 4; }

template <int RT>
__global__ __launch_bounds__(64 * kFacWaves) void tsqr_leaf(FacArgs a) {
  const int lane = threadIdx.x & 63;
  const int job = blockIdx.x * kFacWaves + (threadIdx.x >> 6);
  if (job >= a.M * a.P) return;  // a whole wave
  const int m = job / a.P, l = job - m * a.P;
  const int row0 = l * a.rows_per_leaf, row1 = min(a.d_out, row0 + a.rows_per_leaf);
  const uint16_t *X = a.Bt + int64_t(m) * a.r * a.d_out;  // X[row][c] = X[c * d_out + row]
  constexpr int RPL = leaf_rpl<RT>();
  constexpr int kNew = 64 * RPL - RT;  // new rows per pass
  float x[RPL][RT];
#pragma unroll
  for (int sl = 0; sl < RPL; ++sl)
#pragma unroll
    for (int c = 0; c < RT; ++c) x[sl][c] = 0.f;
  for (int base = row0; base < row1; base += kNew) {
    // new row q: q < 64 - RT in slot 0 of lane RT + q, else in slot
    // 1 + (q - 64 + RT) / 64 of lane (q - 64 + RT) % 64
    // every load is issued (indices clamped into the module) and the
    // invalid ones are replaced afterwards, so the pass waits once for all
    // of them instead of once per guarded load
    // (slots 1.. hold only rows the previous pass zeroed, so they take the
    // loads directly; slot 0 keeps R in lanes < RT and loads into t)
    uint32_t t[RT];
#pragma unroll
    for (int sl = 0; sl < RPL; ++sl) {
      const int gc = min(max(base + 64 * sl + lane - RT, 0), a.d_out - 1);
#pragma unroll
      for (int c = 0; c < RT; ++c) {
        const uint32_t h = X[int64_t(min(c, a.r - 1)) * a.d_out + gc];
        if (sl == 0)
          t[c] = h;
        else
          x[sl][c] = __uint_as_float(h << 16);
      }
    }
#pragma unroll
    for (int sl = 0; sl < RPL; ++sl) {
      const int g = base + 64 * sl + lane - RT;
      const bool ok = (sl > 0 || lane >= RT) && g < row1;
#pragma unroll
      for (int c = 0; c < RT; ++c) {
        if (sl == 0)
          x[0][c] = lane >= RT ? (c < a.r && ok ? __uint_as_float(t[c] << 16) : 0.f) : x[0][c];
        else
          x[sl][c] = c < a.r && ok ? x[sl][c] : 0.f;
      }
    }
    hh_pass<RT, RPL>(x, lane);
  }
  if (lane < RT) {
    float *dst = a.leafR + (int64_t(m) * a.P + l) * RT * RT + lane * RT;
#pragma unroll
    for (int c = 0; c < RT; ++c) dst[c] = x[0][c];
  }
}

// G's share of one column slice: lane (r16, kg) holds Y[16 ib + r16][k0 +
// 8 kg .. + 8] for each 16-row block ib; the block product (ib, jb) is one
// 16x16x32 MFMA whose two operands are the same registers' blocks, and its
// element v of lane (r16, kg) is G[16 ib + 4 kg + v][16 jb + r16].
template <int RT>
__global__ __launch_bounds__(64 * kFacWaves) void gram_kernel(FacArgs a) {
  constexpr int NB = RT / 16;
  const int lane = threadIdx.x & 63, r16 = lane & 15, kg = lane >> 4;
  const int job = blockIdx.x * kFacWaves + (threadIdx.x >> 6);
  if (job >= a.M * a.S) return;
  const int m = job / a.S, s = job - m * a.S;
  const int c0 = s * a.cols_per_split, c1 = min(a.d_in, c0 + a.cols_per_split);
  const uint16_t *Y = a.At + int64_t(m) * a.r * a.d_in;
  ff32x4_t acc[NB][NB];
#pragma unroll
  for (int ib = 0; ib < NB; ++ib)
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) acc[ib][jb] = ff32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = c0; k0 < c1; k0 += 32) {
    const int col = k0 + 8 * kg;  // d_in and the slice bounds are multiples of 8
    fbf16x8_t y[NB];
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      // clamped, unconditional load (c1 - 8 >= c0 is a valid octet), then zero
      const int row = 16 * ib + r16;
      uint4 w = *reinterpret_cast<const uint4 *>(Y + int64_t(min(row, a.r - 1)) * a.d_in +
                                                 min(col, c1 - 8));
      if (!(row < a.r && col < c1)) w = make_uint4(0, 0, 0, 0);
      y[ib] = *reinterpret_cast<const fbf16x8_t *>(&w);
    }
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
        acc[ib][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y[ib], y[jb], acc[ib][jb], 0, 0, 0);
  }
  float *dst = a.gpart + (int64_t(m) * a.S + s) * RT * RT;
#pragma unroll
  for (int ib = 0; ib < NB; ++ib)
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[(16 * ib + 4 * kg + v) * RT + 16 * jb + r16] = acc[ib][jb][v];
}

// Round-robin pairing of RT indices: in round t index 0 meets 1 + t, and for
// i >= 1 the indices 1 + (t + i) and 1 + (t - i) (mod RT - 1) meet.  Every
// round is a perfect matching and RT - 1 rounds meet every pair once.
template <int RT>
__device__ inline void jacobi_pair(int t, int i, int &p, int &q) {
  if (i == 0) {
    p = 0;
    q = 1 + t % (RT - 1);
  } else {
    p = 1 + (t + i) % (RT - 1);
    q = 1 + (t - i + RT - 1) % (RT - 1);
  }
}

constexpr int kCoreThreads = 64;  // one wave per module: barriers are cheap

template <int RT>
__global__ __launch_bounds__(kCoreThreads) void factor_core(FacArgs a) {
  __shared__ double sR[RT][RT + 1], sG[RT][RT + 1], sP[RT][RT + 1], sA[RT][RT + 1], sV[RT][RT + 1];
  __shared__ double rot_c[RT / 2], rot_s[RT / 2], lam[RT];
  __shared__ int perm[RT];
  __shared__ int moved;
  const int tid = threadIdx.x, lane = tid & 63;
  const int m = blockIdx.x;

  {
    // merge the row tiles' R factors: the running R in rows 0..RT-1, the
    // next tile's R in rows RT..2RT-1 (loads clamped, then selected)
    const float *L = a.leafR + int64_t(m) * a.P * RT * RT;
    float x[1][RT];
#pragma unroll
    for (int c = 0; c < RT; ++c) {
      const float v = L[min(lane, RT - 1) * RT + c];
      x[0][c] = lane < RT ? v : 0.f;
    }
    const int li = min(max(lane - RT, 0), RT - 1);
    for (int p = 1; p < a.P; ++p) {
#pragma unroll
      for (int c = 0; c < RT; ++c) {
        const float v = L[(p * RT + li) * RT + c];
        x[0][c] = lane < RT ? x[0][c] : (lane < 2 * RT ? v : 0.f);
      }
      hh_pass<RT, 1>(x, lane);
    }
    if (lane < RT)
#pragma unroll
      for (int c = 0; c < RT; ++c) sR[lane][c] = x[0][c];
    for (int e = tid; e < RT * RT; e += kCoreThreads) {
      double g = 0.0;
      for (int s = 0; s < a.S; ++s) g += a.gpart[(int64_t(m) * a.S + s) * RT * RT + e];
      sG[e / RT][e % RT] = g;
    }
  }
  __syncthreads();
  for (int e = tid; e < RT * RT; e += kCoreThreads) {  // P = R G
    const int i = e / RT, c = e % RT;
    double v = 0.0;
    for (int k = 0; k < RT; ++k) v += sR[i][k] * sG[k][c];
    sP[i][c] = v;
  }
  __syncthreads();
  for (int e = tid; e < RT * RT; e += kCoreThreads) {  // H H^T = P R^T; V = I
    const int i = e / RT, k = e % RT;
    double v = 0.0;
    for (int c = 0; c < RT; ++c) v += sP[i][c] * sR[k][c];
    sA[i][k] = v;
    sV[i][k] = i == k ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int e = tid; e < RT * RT; e += kCoreThreads) {  // exact symmetry
    const int i = e / RT, k = e % RT;
    if (i < k) {
      const double v = 0.5 * (sA[i][k] + sA[k][i]);
      sA[i][k] = v;
      sA[k][i] = v;
    }
  }
  __syncthreads();

  // cyclic Jacobi, RT / 2 disjoint rotations per round: A <- J^T A J, V <- V J
  for (int sw = 0; sw < kJacobiSweeps; ++sw) {
    if (tid == 0) moved = 0;
    __syncthreads();
    for (int t = 0; t < RT - 1; ++t) {
      if (tid < RT / 2) {
        int p, q;
        jacobi_pair<RT>(t, tid, p, q);
        const double apq = sA[p][q], app = sA[p][p], aqq = sA[q][q];
        double c = 1.0, s = 0.0;
        if (fabs(apq) > 0x1p-52 * sqrt(fabs(app * aqq))) {
          const double tau = (aqq - app) / (2.0 * apq);
          const double tt = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + tt * tt);
          s = tt * c;
          moved = 1;
        }
        rot_c[tid] = c;
        rot_s[tid] = s;
      }
      __syncthreads();
      // J^T A J by 2 x 2 blocks: block (i, k) holds rows (p_i, q_i) and
      // columns (p_k, q_k); rotating its rows by pair i, then its columns
      // by pair k, touches no other block.  The rotated pair's own (p, q)
      // entries are stored as exact zeros.  V <- V J in the same pass.
      for (int e = tid; e < RT / 2 * RT / 2; e += kCoreThreads) {
        const int i = e / (RT / 2), k = e % (RT / 2);
        int pi, qi, pk, qk;
        jacobi_pair<RT>(t, i, pi, qi);
        jacobi_pair<RT>(t, k, pk, qk);
        const double ci = rot_c[i], si = rot_s[i], ck = rot_c[k], sk = rot_s[k];
        const double a0 = sA[pi][pk], b0 = sA[pi][qk], c0 = sA[qi][pk], d0 = sA[qi][qk];
        const double a1 = ci * a0 - si * c0, b1 = ci * b0 - si * d0;
        const double c1 = si * a0 + ci * c0, d1 = si * b0 + ci * d0;
        sA[pi][pk] = ck * a1 - sk * b1;
        sA[pi][qk] = i == k ? 0.0 : sk * a1 + ck * b1;
        sA[qi][pk] = i == k ? 0.0 : ck * c1 - sk * d1;
        sA[qi][qk] = sk * c1 + ck * d1;
      }
      for (int e = tid; e < RT * RT / 2; e += kCoreThreads) {
        const int row = e / (RT / 2), k = e % (RT / 2);
        int pk, qk;
        jacobi_pair<RT>(t, k, pk, qk);
        const double ck = rot_c[k], sk = rot_s[k], vp = sV[row][pk], vq = sV[row][qk];
        sV[row][pk] = ck * vp - sk * vq;
        sV[row][qk] = sk * vp + ck * vq;
      }
      __syncthreads();
    }
    const int mv = moved;
    __syncthreads();
    if (!mv) break;
  }

  if (tid < RT) lam[tid] = sA[tid][tid];
  __syncthreads();
  if (tid < RT) {
    const double l = lam[tid];
    int rank = 0;
    for (int i = 0; i < RT; ++i) rank += lam[i] > l || (lam[i] == l && i < tid);
    perm[rank] = tid;
  }
  __syncthreads();
  double lmax = 0.0;
  for (int i = 0; i < RT; ++i) lmax = fmax(lmax, lam[i]);
  float *Mf = a.mats + int64_t(m) * 2 * RT * RT, *Mt = Mf + RT * RT;
  for (int e = tid; e < RT * RT; e += kCoreThreads) {
    const int pos = e / RT, c = e % RT, j = perm[pos];
    const double l = lam[j];
    const bool live = lmax > 0.0 && l > 0x1p-23 * lmax;
    double mt = 0.0, mf = 0.0, sg = 0.0;
    if (live) {
      sg = sqrt(l);
      for (int i = 0; i < RT; ++i) {
        mt += sV[i][j] * sR[i][c];
        mf += sV[i][j] * sP[i][c];
      }
      const double rs = sqrt(sg);
      mt /= rs;
      mf /= sg * rs;
    }
    Mf[pos * RT + c] = float(mf);
    Mt[pos * RT + c] = float(mt);
    if (c == 0 && pos < a.r) a.sigma[int64_t(m) * a.r + pos] = float(sg);
  }
}

// F^T rows (z = 0: from B_t, map Mf) or T rows (z = 1: from A_t, map Mt);
// one thread per pair of columns.
template <int RT>
__global__ __launch_bounds__(256) void factor_out(FacArgs a) {
  __shared__ float sM[RT][RT];
  const int m = blockIdx.y, which = blockIdx.z;
  const int D = which ? a.d_in : a.d_out;
  const float *Mm = a.mats + (int64_t(m) * 2 + which) * RT * RT;
  for (int e = threadIdx.x; e < RT * RT; e += 256) sM[e / RT][e % RT] = Mm[e];
  __syncthreads();
  const int n = (blockIdx.x * 256 + threadIdx.x) * 2;  // D is even
  if (n >= D) return;
  const uint16_t *In = (which ? a.At : a.Bt) + int64_t(m) * a.r * D;
  uint16_t *Out = (which ? a.T : a.Ft) + int64_t(m) * a.r * D;
  float in0[RT], in1[RT];
#pragma unroll
  for (int c = 0; c < RT; ++c) {
    uint32_t w = *reinterpret_cast<const uint32_t *>(In + int64_t(min(c, a.r - 1)) * D + n);
    if (c >= a.r) w = 0;
    in0[c] = __uint_as_float(w << 16);
    in1[c] = __uint_as_float(w & 0xffff0000u);
  }
#pragma unroll
  for (int pos = 0; pos < RT; ++pos) {
    if (pos < a.r) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int c = 0; c < RT; ++c) {
        s0 += sM[pos][c] * in0[c];
        s1 += sM[pos][c] * in1[c];
      }
      *reinterpret_cast<uint32_t *>(Out + int64_t(pos) * D + n) =
          uint32_t(to_bf16(s0)) | (uint32_t(to_bf16(s1)) << 16);
    }
  }
}

struct FacGeom {
  int RT, P, S, rows_per_leaf, cols_per_split;
  size_t off_leaf, off_gram, off_mats, bytes;
};

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int factor_geometry(int32_t M, int32_t d_out, int32_t d_in, int32_t r, FacGeom &g) {
  if (M < 0) return fail(TCL_EINVAL, "factor: n_modules %d < 0", M);
  if (M > 65535) return fail(TCL_EINVAL, "factor: n_modules %d > 65535", M);
  if (r < 1 || r > kFacMaxRank) return fail(TCL_EUNSUPPORTED, "factor: rank %d outside 1..%d", r, kFacMaxRank);
  if (d_out < 2 || d_in < 8) return fail(TCL_EINVAL, "factor: d_out %d < 2 or d_in %d < 8", d_out, d_in);
  if (d_out % 2 || d_in % 8)
    return fail(TCL_EALIGN, "factor: d_out must be even and d_in a multiple of 8 (%d, %d)", d_out, d_in);
  g.RT = r <= 16 ? 16 : 32;
  const int kNew = 64 * (g.RT == 16 ? leaf_rpl<16>() : leaf_rpl<32>()) - g.RT;  // leaf rows per pass
  const int Mm = std::max(M, 1);
  int P = std::max(1, std::min((kLeafWaveTarget + Mm - 1) / Mm, kMaxLeaves));
  P = std::min(P, (d_out + kNew - 1) / kNew);
  g.rows_per_leaf = ((d_out + P - 1) / P + kNew - 1) / kNew * kNew;
  g.P = (d_out + g.rows_per_leaf - 1) / g.rows_per_leaf;
  int S = std::max(1, (kGramWaveTarget + Mm - 1) / Mm);
  S = std::min(S, std::max(1, d_in / 256));
  g.cols_per_split = ((d_in + S - 1) / S + 31) / 32 * 32;
  g.S = (d_in + g.cols_per_split - 1) / g.cols_per_split;
  if (int64_t(M) * g.P >= (int64_t(1) << 30) || int64_t(M) * g.S >= (int64_t(1) << 30))
    return fail(TCL_EINVAL, "factor: batch too large");
  const size_t tile = size_t(g.RT) * g.RT * sizeof(float);
  g.off_leaf = 0;
  g.off_gram = round256(size_t(M) * g.P * tile);
  g.off_mats = g.off_gram + round256(size_t(M) * g.S * tile);
  g.bytes = g.off_mats + round256(size_t(M) * 2 * tile);
  return TCL_OK;
}

template <int RT>
void launch_factor(const FacArgs &a, hipStream_t st) {
  const int64_t leaf_waves = int64_t(a.M) * a.P, gram_waves = int64_t(a.M) * a.S;
  hipLaunchKernelGGL(tsqr_leaf<RT>, dim3(unsigned((leaf_waves + kFacWaves - 1) / kFacWaves)),
                     dim3(64 * kFacWaves), 0, st, a);
  hipLaunchKernelGGL(gram_kernel<RT>, dim3(unsigned((gram_waves + kFacWaves - 1) / kFacWaves)),
                     dim3(64 * kFacWaves), 0, st, a);
  hipLaunchKernelGGL(factor_core<RT>, dim3(a.M), dim3(kCoreThreads), 0, st, a);
  const int D = std::max(a.d_out, a.d_in);
  hipLaunchKernelGGL(factor_out<RT>, dim3((D / 2 + 255) / 256, a.M, 2), dim3(256), 0, st, a);
}

}  // namespace
}  // namespace tcl

using namespace tcl;

extern "C" int tcl_factor_workspace_bytes(int32_t n_modules, int32_t d_out, int32_t d_in,
                                          int32_t rank, size_t *bytes) {
  if (!bytes) return fail(TCL_EINVAL, "factor: bytes is NULL");
  FacGeom g;
  if (int rc = factor_geometry(n_modules, d_out, d_in, rank, g)) return rc;
  *bytes = g.bytes;
  return TCL_OK;
}

extern "C" int tcl_factor_balanced(const void *B_t, const void *A_t, int32_t n_modules,
                                   int32_t d_out, int32_t d_in, int32_t rank, void *F_t, void *T,
                                   float *sigma, void *ws, size_t ws_bytes, void *stream) {
  FacGeom g;
  if (int rc = factor_geometry(n_modules, d_out, d_in, rank, g)) return rc;
  if (n_modules == 0) return TCL_OK;
  if (!B_t || !A_t || !F_t || !T || !sigma || !ws) return fail(TCL_EINVAL, "factor: NULL pointer");
  if ((reinterpret_cast<uintptr_t>(A_t) | reinterpret_cast<uintptr_t>(ws)) & 15)
    return fail(TCL_EALIGN, "factor: A_t and ws must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(B_t) | reinterpret_cast<uintptr_t>(F_t) |
       reinterpret_cast<uintptr_t>(T) | reinterpret_cast<uintptr_t>(sigma)) & 3)
    return fail(TCL_EALIGN, "factor: B_t, F_t, T and sigma must be 4-byte aligned");
  if (ws_bytes < g.bytes) return fail(TCL_ENOSPC, "factor: workspace %zu < %zu bytes", ws_bytes, g.bytes);
  char *w = static_cast<char *>(ws);
  FacArgs a{static_cast<const uint16_t *>(B_t), static_cast<const uint16_t *>(A_t),
            static_cast<uint16_t *>(F_t), static_cast<uint16_t *>(T), sigma,
            reinterpret_cast<float *>(w + g.off_leaf), reinterpret_cast<float *>(w + g.off_gram),
            reinterpret_cast<float *>(w + g.off_mats), n_modules, d_out, d_in, rank, g.P, g.S,
            g.rows_per_leaf, g.cols_per_split};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (g.RT == 16)
    launch_factor<16>(a, st);
  else
    launch_factor<32>(a, st);
  TCL_HIP(hipGetLastError());
  return TCL_OK;
}

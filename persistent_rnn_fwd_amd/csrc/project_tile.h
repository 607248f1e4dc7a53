// One workgroup's tile of an input projection on the matrix cores:
//
//   X[m][n] = bias[n] + sum_i U[n][i] * x[m][i]
//
// ("Optimizing Performance of Recurrent Neural Networks on GPUs", Abstract,
// single-layer stage: the input-side product of every timestep does not
// depend on the state, so it is one matrix product ahead of the recurrence.)
//
// Products are v_mfma_f32_16x16x32_f16 with fp32 accumulation.  fp32 x enters
// as two fp16 operands: hi is x with the low 13 bits of its fp32 significand
// cleared (11 significant bits, so exact in fp16 for 2^-14 <= |x| < 2^16) and
// lo = fp16(x - hi), the difference being exact in fp32.  Both products with
// the fp16 U are exact in the accumulators, so x is seen to about 2^-22 of
// |x| (below 2^-14, to about 2^-25 absolute).  |x| >= 2^16, infinities
// included, would make hi overflow fp16 and is reported as a range failure; a
// NaN x passes on as NaN.  fp16 x enters as it is.
//
// The tile is 64 rows of x by BN = 128 or 64 rows of U, computed by 512
// threads in two groups of 4 waves, each over one half of the k range (more
// loads in flight per CU; the two partial tiles are added in a fixed order at
// the end, through LDS).  Within a group, wave (wy, wx) computes a 32 x BN/2
// quarter as 2 x BN/32 MFMA tiles.  Per 32-wide k-step a group stages x (split
// into hi and lo) and U in LDS as fp16 rows of 32 values padded to 48 (a
// 96-byte stride, the fastest of the strides 80 to 144 bytes measured at the
// layer size), double buffered, so one barrier per k-step separates writing
// a buffer from reading it; global loads run DEPTH k-steps ahead of the
// products.  Each wave reads its operands straight in the MFMA layout (lane
// l: row l % 16, values 8 (l / 16) .. + 7 of the k-step): 8 LDS reads feed 16
// products, the 8 hi products first so that no product waits for the one
// before it.  The k range, its split over the groups and the order of the
// products depend only on I and DEPTH, so every tile computes an element of X
// the same way wherever the tile lies.
//
// Tile row m lies at row m * stride + offset of x ([..][I]) and of X
// ([..][ldx]): the plain projection uses stride 1, a block of one batch row
// of a [T][B][.] sequence stride B and offset b.  Rows past the end of x's
// buffer read zeros (buffer bounds), and only rows m < M and columns
// n < n_end of X are stored.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace prnn {
namespace proj {

typedef _Float16 ph8 __attribute__((ext_vector_type(8)));
typedef float pf4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;        // rows of x per tile (rows of U: BN = 128 or 64)
constexpr int kRow = 48;       // fp16 per LDS row (32 + 16 padding; the fastest of 40-72, measured)
template <int BN>
constexpr int stage_halves() { return (2 * kBM + BN) * kRow; }  // fp16 per buffer: x hi, x lo, U
constexpr int kGroups = 2;                      // k-range halves per workgroup, 4 waves each
constexpr int kThreads = 256 * kGroups;
constexpr int kDepth = 4;                       // k-steps of global loads in flight (default)
// LDS of one tile: both groups' double buffers (the final reduction reuses it)
template <int BN>
constexpr int lds_bytes() { return kGroups * 2 * stage_halves<BN>() * 2; }

// Offset past every buffer here (the host keeps x and U below 0xFFFFFF00
// bytes): a load from it returns zeros without touching memory.
constexpr uint32_t kOutside = 0xFFFFFFE0u;

// Where tile row m lies in x and X (see the file comment).
struct TileRows {
  int M;       // rows in the tile set: m < M are stored
  int stride;  // row of x and X = m * stride + offset
  int offset;
};

// 8 consecutive values of one row starting at column k, as raw words (8 fp32
// in w0, w1; or 8 fp16 in w0).  Rows past the end read 0 (buffer bounds);
// columns past I read 0 through kOutside.  No branches: a branch around a
// load makes the compiler wait for every load in flight where it rejoins.
template <bool F32, bool VEC>
__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t r, int row, int k, int I, u32x4& w0, u32x4& w1) {
  constexpr uint32_t esize = F32 ? 4u : 2u;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if (VEC) {
    // I % 8 == 0: the 8 values are all inside the row or all past its end.
    const uint32_t off = k < I ? ((uint32_t)row * (uint32_t)I + (uint32_t)k) * esize : kOutside;
    w0 = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPlain);
    w1 = F32 ? __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u, 0, kPlain) : zero;
    return;
  }
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t off = k + e < I ? ((uint32_t)row * (uint32_t)I + (uint32_t)(k + e)) * esize : kOutside;
    if (F32)
      v[e] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kPlain);
    else
      v[e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kPlain);
  }
  if (F32) {
    w0 = u32x4{v[0], v[1], v[2], v[3]};
    w1 = u32x4{v[4], v[5], v[6], v[7]};
  } else {
    w0 = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
    w1 = zero;
  }
}

// fp32 words -> hi and lo fp16 (see the file comment); `amax` keeps the
// largest |x| seen (NaNs do not count), tested against 2^16 once at the end.
__device__ __forceinline__ void split8(const u32x4& w0, const u32x4& w1, ph8& hi, ph8& lo, float& amax) {
  const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = __uint_as_float(w[e]);
    const float h = __uint_as_float(w[e] & 0xFFFFE000u);
    hi[e] = (_Float16)h;               // exact where in range
    lo[e] = (_Float16)(f - h);         // f - h is exact in fp32
    amax = __builtin_fmaxf(amax, __builtin_fabsf(f));
  }
}

// This thread's share of one k-step's global operands: 8 values of x (tile
// row t / 4, columns 8 (t % 4)) and of U 16 values (BN = 128: row t / 2,
// columns 16 (t % 2)) or 8 (BN = 64: row t / 4, columns 8 (t % 4)).
struct Staged {
  u32x4 x0, x1, u0, u1;
};

template <bool XF32, bool VEC, int BN>
__device__ __forceinline__ void fetch(Staged& s, __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t ur,
                                      const TileRows& rows, int mb, int nb, int k0, int I, int t) {
  u32x4 none;
  load8<XF32, VEC>(xr, (mb + (t >> 2)) * rows.stride + rows.offset, k0 + 8 * (t & 3), I, s.x0, s.x1);
  if (BN == 128) {
    load8<false, VEC>(ur, nb + (t >> 1), k0 + 16 * (t & 1), I, s.u0, none);
    load8<false, VEC>(ur, nb + (t >> 1), k0 + 16 * (t & 1) + 8, I, s.u1, none);
  } else {
    load8<false, VEC>(ur, nb + (t >> 2), k0 + 8 * (t & 3), I, s.u0, none);
  }
}

template <bool XF32, int BN>
__device__ __forceinline__ void stage(const Staged& s, _Float16* buf, int t, float& amax) {
  _Float16* xhi = buf;
  _Float16* xlo = buf + kBM * kRow;
  _Float16* u = buf + 2 * kBM * kRow;
  const int xo = (t >> 2) * kRow + 8 * (t & 3);
  if (XF32) {
    ph8 hi, lo;
    split8(s.x0, s.x1, hi, lo, amax);
    *reinterpret_cast<ph8*>(xhi + xo) = hi;
    *reinterpret_cast<ph8*>(xlo + xo) = lo;
  } else {
    *reinterpret_cast<u32x4*>(xhi + xo) = s.x0;
  }
  if (BN == 128) {
    const int uo = (t >> 1) * kRow + 16 * (t & 1);
    *reinterpret_cast<u32x4*>(u + uo) = s.u0;
    *reinterpret_cast<u32x4*>(u + uo + 8) = s.u1;
  } else {
    *reinterpret_cast<u32x4*>(u + (t >> 2) * kRow + 8 * (t & 3)) = s.u0;
  }
}

// The 64 x BN tile of X at tile rows [mb, mb + 64) and U rows [nb, nb + BN),
// by all 512 threads of the workgroup (uniform control flow: every thread
// calls it and passes the same barriers).  `lds_all` holds lds_bytes<BN>()
// bytes; it is free again when the call returns.  Returns false in a thread
// that staged an fp32 x with |x| >= 2^16 (or infinite).
template <bool XF32, bool VEC, int BN, int DEPTH = kDepth>
__device__ __forceinline__ bool project_tile(__amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t ur, const float* bias,
                                             float* X, int ldx, const TileRows& rows, int mb, int nb, int n_end,
                                             int I, _Float16* lds_all) {
  constexpr int kStage = stage_halves<BN>();
  constexpr int TN = BN / 32;  // 16-column MFMA tiles per wave
  const int grp = threadIdx.x >> 8;
  const int t = threadIdx.x & 255;  // thread within the group
  _Float16* lds = lds_all + grp * 2 * kStage;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int wy = wave >> 1, wx = wave & 1;

  pf4 acc[2][TN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = pf4{0.f, 0.f, 0.f, 0.f};
  float amax = 0.f;  // largest |x| staged by this thread

  // This group's k-steps: [grp * half, grp * half + half), half a multiple
  // of DEPTH.  Steps past the end of the row load zeros and add exactly
  // nothing, so both groups run the same number of steps (and barriers).
  const int half = ((((I + 31) / 32 + kGroups - 1) / kGroups) + DEPTH - 1) / DEPTH * DEPTH;
  const int kbase = 32 * half * grp;
  // Global loads run DEPTH k-steps ahead of the products, in DEPTH register
  // sets used in turn (set k % DEPTH holds step k; an in-flight set is never
  // copied, which would wait for it).
  Staged st[DEPTH];
  fetch<XF32, VEC, BN>(st[0], xr, ur, rows, mb, nb, kbase, I, t);
  stage<XF32, BN>(st[0], lds, t, amax);
#pragma unroll
  for (int d = 1; d <= DEPTH; ++d) fetch<XF32, VEC, BN>(st[d % DEPTH], xr, ur, rows, mb, nb, kbase + 32 * d, I, t);
  __syncthreads();

  auto step = [&](int kk, Staged& next) {
    const _Float16* buf = lds + (kk & 1) * kStage;
    ph8 ahi[2], alo[2], b[TN];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = (32 * wy + 16 * i + r16) * kRow + 8 * q;
      ahi[i] = *reinterpret_cast<const ph8*>(buf + o);
      if (XF32) alo[i] = *reinterpret_cast<const ph8*>(buf + kBM * kRow + o);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = *reinterpret_cast<const ph8*>(buf + 2 * kBM * kRow + ((BN / 2) * wx + 16 * j + r16) * kRow + 8 * q);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[i], b[j], acc[i][j], 0, 0, 0);
    if (XF32) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[i], b[j], acc[i][j], 0, 0, 0);
    }
    // `next` holds step kk + 1: into the other buffer, then reload it with
    // step kk + 1 + DEPTH.  Past the group's last step these load zeros and
    // fill a buffer nobody reads (no branch, see load8).
    stage<XF32, BN>(next, lds + ((kk + 1) & 1) * kStage, t, amax);
    fetch<XF32, VEC, BN>(next, xr, ur, rows, mb, nb, kbase + 32 * (kk + 1 + DEPTH), I, t);
    __syncthreads();
  };
  for (int kk = 0; kk < half; kk += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(kk + d, st[(d + 1) % DEPTH]);
  }

  // The second group's partial tile onto the first's: X = first + second.
  float* red = reinterpret_cast<float*>(lds_all);  // [4 waves][2 TN tiles x 4][64 lanes]
  if (grp == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(wave * 8 * TN + (i * TN + j) * 4 + r) * 64 + lane] = acc[i][j][r];
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] += red[(wave * 8 * TN + (i * TN + j) * 4 + r) * 64 + lane];

    // D layout: lane holds rows 4 q .. 4 q + 3 of column r16 of each 16 x 16 tile.
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = nb + (BN / 2) * wx + 16 * j + r16;
      if (n >= n_end) continue;
      const float bn = bias != nullptr ? bias[n] : 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mb + 32 * wy + 16 * i + 4 * q + r;
          if (m < rows.M) X[(size_t)(m * rows.stride + rows.offset) * ldx + n] = acc[i][j][r] + bn;
        }
    }
  }
  __syncthreads();  // the reduction area is read before anyone reuses the LDS
  return !(amax >= 65536.f);
}

}  // namespace proj
}  // namespace prnn

// Elementwise and data-movement kernels of the POET layer: skew packing, the skew projection of the
// gradient, FS index gather/scatter, dtype conversion, and the counter-based FS index sampler.
// All are memory-bound; threads walk the contiguous dimension so that every wavefront access is coalesced.
#include <algorithm>

#include "../../include/poet.h"
#include "internal.h"

namespace poet {
namespace {

constexpr int kThreads = 256;

inline int grid_for(size_t n, int per_block = kThreads, int cap = 65535 * 8) {
  size_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g > (size_t)cap ? cap : g);
}


// Q of one 32 x 32 tile pair of a primitive from its packed parameters. Workgroup (256 threads) = tile pair
// (ti, tj), ti <= tj, of primitive p; thread (col = tid % 32, row0 = tid / 32) holds rows row0 + 8u, u = 0..3.
// up[u] = Q(32 ti + r, 32 tj + col) (upper tile, read row-wise from the packed strict upper triangle: coalesced),
// lo[u] = Q(32 tj + r, 32 ti + col) = -Q(32 ti + col, 32 tj + r) (the transpose, through LDS). On a diagonal tile
// (ti == tj) up holds the whole tile and lo is unused.
__device__ __forceinline__ void tile_pair_of(int tpair, int bp, int& ti, int& tj) {
  const int nt = (bp + 31) / 32;
  int rem = tpair;
  ti = 0;
  while (rem >= nt - ti) { rem -= nt - ti; ++ti; }
  tj = ti + rem;
}
__device__ __forceinline__ void q_tile_pair(const float* __restrict__ theta, int64_t toff, int c, int ti, int tj,
                                            float (*tr)[33], float up[4], float lo[4]) {
  const int col = threadIdx.x & 31, row0 = threadIdx.x >> 5;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = row0 + 8 * u, i = ti * 32 + r, j = tj * 32 + col;
    up[u] = (i < j && j < c) ? theta[toff + tri_pos(i, j, c)] : 0.f;
    tr[r][col] = up[u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = row0 + 8 * u;
    if (ti == tj) {
      if (r > col) up[u] = -tr[col][r];  // the lower half of a diagonal tile
      lo[u] = 0.f;
    } else {
      lo[u] = -tr[col][r];
    }
  }
}

// Q at row r, column cc of half h of a tile pair from the staged upper tile tr (zero at and below the diagonal
// and past the primitive's size): h = 0 the tile (ti, tj), h = 1 its mirror (tj, ti) = -(ti, tj)^T; below the
// diagonal of a diagonal tile, minus the transposed element (the values q_tile_pair gives, signed zeros included)
__device__ __forceinline__ float q_of(const float (*tr)[33], int h, bool diag, int r, int cc) {
  return (h || (diag && r > cc)) ? -tr[cc][r] : tr[r][cc];
}

// V consecutive elements of a row as one load or store (V = 4, 2 or 1; the caller checks alignment)
template <int V>
__device__ __forceinline__ void ld_row(const void* p, int dt, int64_t i, float (&o)[V]) {
  if (dt == BF16) {
    const __bf16* b = reinterpret_cast<const __bf16*>(p) + i;
    if constexpr (V == 4) {
      typedef __bf16 v4 __attribute__((ext_vector_type(4)));
      const v4 x = *reinterpret_cast<const v4*>(b);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (float)x[e];
    } else if constexpr (V == 2) {
      typedef __bf16 v2 __attribute__((ext_vector_type(2)));
      const v2 x = *reinterpret_cast<const v2*>(b);
      o[0] = (float)x[0]; o[1] = (float)x[1];
    } else {
      o[0] = (float)b[0];
    }
  } else {
    const float* f = reinterpret_cast<const float*>(p) + i;
    if constexpr (V == 4) {
      const float4 x = *reinterpret_cast<const float4*>(f);
      o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    } else if constexpr (V == 2) {
      const float2 x = *reinterpret_cast<const float2*>(f);
      o[0] = x.x; o[1] = x.y;
    } else {
      o[0] = f[0];
    }
  }
}
template <int V>
__device__ __forceinline__ void st_row(void* p, int dt, int64_t i, const float (&v)[V]) {
  if (dt == BF16) {
    __bf16* b = reinterpret_cast<__bf16*>(p) + i;
    if constexpr (V == 4) {
      typedef __bf16 v4 __attribute__((ext_vector_type(4)));
      v4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (__bf16)v[e];
      *reinterpret_cast<v4*>(b) = x;
    } else if constexpr (V == 2) {
      typedef __bf16 v2 __attribute__((ext_vector_type(2)));
      v2 x;
      x[0] = (__bf16)v[0]; x[1] = (__bf16)v[1];
      *reinterpret_cast<v2*>(b) = x;
    } else {
      b[0] = (__bf16)v[0];
    }
  } else {
    float* f = reinterpret_cast<float*>(p) + i;
    if constexpr (V == 4) *reinterpret_cast<float4*>(f) = make_float4(v[0], v[1], v[2], v[3]);
    else if constexpr (V == 2) *reinterpret_cast<float2*>(f) = make_float2(v[0], v[1]);
    else f[0] = v[0];
  }
}

// prim = I + coef Q and the first saved power Q (dtype q_dt, row pitch ldq) of side blockIdx.z of the table,
// primitive blockIdx.y, tile pair blockIdx.x. A thread takes V consecutive columns of a row (32 / V threads per tile
// row), so prim and Q leave as V-element stores where the row holds them.
template <int V>
__global__ __launch_bounds__(256) void k_theta_prep(const PrepGroup G) {
  __shared__ float tr[32][33];
  PrepSide a;
  {
    const PrepSide& t = G.s[blockIdx.z];
    a.theta = keep_s(t.theta); a.prim = keep_s(t.prim); a.q = keep_s(t.q); a.q_dt = keep_s(t.q_dt);
    a.ldq = keep_s(t.ldq); a.mode = keep_s(t.mode); a.d = keep_s(t.d); a.bp = keep_s(t.bp);
    a.nprim = keep_s(t.nprim); a.coef = keep_s(t.coef);
  }
  const int bp = a.bp, p = blockIdx.y, nt = (bp + 31) / 32;
  if (p >= a.nprim || (int)blockIdx.x >= nt * (nt + 1) / 2) return;
  int ti, tj;
  tile_pair_of(blockIdx.x, bp, ti, tj);
  const int c = prim_size(a.mode, a.d, bp, p);
  float up[4], lo[4];
  q_tile_pair(a.theta, theta_off(bp, p), c, ti, tj, tr, up, lo);  // stages the upper tile in tr
  constexpr int TPR = 32 / V, RPP = 256 / TPR;
  const int cv = (threadIdx.x % TPR) * V, r0 = threadIdx.x / TPR;
  const bool diag = ti == tj;
  float* prim = a.prim + (int64_t)p * bp * bp;
  for (int h = 0; h < 2; ++h) {
    if (h == 1 && diag) break;
    const int ri = h ? tj : ti, cj = h ? ti : tj;
    for (int r = r0; r < 32; r += RPP) {
      const int i = ri * 32 + r, j0 = cj * 32 + cv;
      if (i >= bp || j0 >= bp) continue;
      const int64_t e0 = (int64_t)i * bp + j0, o0 = ((int64_t)p * bp + i) * a.ldq + j0;
      if (j0 + V <= bp) {
        float q[V], pv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          q[e] = q_of(tr, h, diag, r, cv + e);
          pv[e] = (i == j0 + e ? 1.f : 0.f) + a.coef * q[e];
        }
        st_row<V>(prim, F32, e0, pv);
        if (a.q) st_row<V>(a.q, a.q_dt, o0, q);
      } else {  // the last columns of a ragged block, one at a time
        for (int e = 0; e < V && j0 + e < bp; ++e) {
          const float q = q_of(tr, h, diag, r, cv + e);
          prim[e0 + e] = (i == j0 + e ? 1.f : 0.f) + a.coef * q;
          if (a.q) {
            if (a.q_dt == BF16) reinterpret_cast<__bf16*>(a.q)[o0 + e] = (__bf16)q;
            else reinterpret_cast<float*>(a.q)[o0 + e] = q;
          }
        }
      }
    }
  }
}

__global__ void k_qnorm(const float* __restrict__ theta, int mode, int d, int bp, float* __restrict__ qnorm) {
  __shared__ float red[kThreads];
  const int p = blockIdx.x;
  const int c = prim_size(mode, d, bp, p);
  const int64_t off = theta_off(bp, p), n = (int64_t)c * (c - 1) / 2;
  float s = 0.f;
  for (int64_t t = threadIdx.x; t < n; t += kThreads) {
    const float v = theta[off + t];
    s += v * v;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) qnorm[p] = sqrtf(2.f * red[0]);
}

__global__ void k_skew_project(const float* __restrict__ dQ, const float* __restrict__ G1, int mode, int d,
                               int bp, int nprim, float* __restrict__ dtheta) {
  const int64_t total = (int64_t)nprim * bp * bp;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(e / ((int64_t)bp * bp));
    const int rem = (int)(e - (int64_t)p * bp * bp);
    const int i = rem / bp, j = rem % bp;
    const int c = prim_size(mode, d, bp, p);
    if (i < j && j < c) {
      const int64_t base = (int64_t)p * bp * bp;
      const int64_t ij = base + (int64_t)i * bp + j, ji = base + (int64_t)j * bp + i;
      float a = dQ[ij], b = dQ[ji];
      if (G1) { a += G1[ij]; b += G1[ji]; }
      dtheta[theta_off(bp, p) + tri_pos(i, j, c)] = a - b;
    }
  }
}

// dtheta of primitive p = blockIdx.y of side blockIdx.z from NS split-K partials: X = sum_s part[s] (split order) +
// beta D, then X_ij - X_ji. The side's blocks sit at block offset boff of the partials (split stride split_stride).
// Workgroup x takes the pair of 32 x 32 tiles (ti, tj), ti <= tj: both are read row-wise (coalesced, the NS loads
// of a thread issued together), the (tj, ti) tile is transposed through LDS.
template <int NS>
__global__ __launch_bounds__(256) void k_reduce_skew(const SkewGroup G) {
  __shared__ float tr[32][33];
  SkewSide a;
  {
    const SkewSide& t = G.s[blockIdx.z];
    a.D = keep_s(t.D); a.dtheta = keep_s(t.dtheta); a.mode = keep_s(t.mode); a.d = keep_s(t.d);
    a.nprim = keep_s(t.nprim); a.boff = keep_s(t.boff);
  }
  const int p = blockIdx.y;
  if (p >= a.nprim) return;
  const int bp = G.bp;
  int ti = 0, rem = blockIdx.x;  // blockIdx.x enumerates ti <= tj row by row
  const int nt = (bp + 31) / 32;
  while (rem >= nt - ti) { rem -= nt - ti; ++ti; }
  const int tj = ti + rem;
  const int c = prim_size(a.mode, a.d, bp, p);
  const int64_t base = (int64_t)p * bp * bp;
  const float* part = G.part + (int64_t)a.boff * bp * bp;
  const int64_t split_stride = G.split_stride;
  const int col = threadIdx.x & 31, row0 = threadIdx.x >> 5;  // rows row0 + 8 q
  float xa[4], xb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = row0 + 8 * q;
    const int ia = ti * 32 + r, ja = tj * 32 + col;  // element of tile (ti, tj)
    const int ib = tj * 32 + r, jb = ti * 32 + col;  // element of tile (tj, ti)
    const bool ina = ia < bp && ja < bp, inb = ib < bp && jb < bp;
    const int64_t oa = base + (ina ? (int64_t)ia * bp + ja : 0), ob = base + (inb ? (int64_t)ib * bp + jb : 0);
    float va[NS], vb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      va[s] = part[s * split_stride + oa];
      vb[s] = part[s * split_stride + ob];
    }
    xa[q] = va[0];
    xb[q] = vb[0];
#pragma unroll
    for (int s = 1; s < NS; ++s) {
      xa[q] += va[s];
      xb[q] += vb[s];
    }
    if (a.D) {
      xa[q] += G.beta * a.D[oa];
      xb[q] += G.beta * a.D[ob];
    }
    tr[col][r] = xb[q];  // transposed: tr[jb - 32 ti][ib - 32 tj]
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = row0 + 8 * q;
    const int i = ti * 32 + r, j = tj * 32 + col;
    if (i < j && j < c) a.dtheta[theta_off(bp, p) + tri_pos(i, j, c)] = xa[q] - tr[r][col];
  }
}

__global__ void k_fill(float* __restrict__ p, size_t n, float v) {
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) p[e] = v;
}

// grid (x, entries): blocks of column y fill entry y
__global__ void k_fill_group(const FillGroup G, float v) {
  const FillEntry& ge = G.a[blockIdx.y];
  float* p = keep_s(ge.p);
  const size_t n = keep_s(ge.n);
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) p[e] = v;
}

__device__ __forceinline__ int clampi(int v, int lim) { return v < 0 ? 0 : (v >= lim ? lim - 1 : v); }

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// Row copies from float32, four consecutive elements per thread: dst[dr][c] = src[sr][c] (dst float32 or bf16) and,
// when dst2 is given, dst2[dr][c] = bf16(src[sr][c]), for rows i < rows with sr = sidx[i] (gather) or i, dr =
// didx[i] (scatter) or i. vec: every pitch a multiple of 4 elements and every base 16-byte aligned, so whole
// groups of four move as one 16-byte load and one 16- or 8-byte store; the row's last partial group goes
// element by element.
__global__ __launch_bounds__(256) void k_rows4(const float* __restrict__ src, int64_t ld_src,
                                               const int32_t* __restrict__ sidx, const int32_t* __restrict__ didx,
                                               int dlim, int rows, int cols, void* __restrict__ dst, int dst_dt,
                                               int64_t ld_dst, __bf16* __restrict__ dst2, int64_t ld_dst2, int vec) {
  for (int i = blockIdx.y; i < rows; i += gridDim.y) {
    const int64_t sr = sidx ? clampi(sidx[i], dlim) : i, dr = didx ? clampi(didx[i], dlim) : i;
    const float* srow = src + sr * ld_src;
    for (int c = 4 * (blockIdx.x * blockDim.x + threadIdx.x); c < cols; c += 4 * gridDim.x * blockDim.x) {
      if (vec && c + 4 <= cols) {
        const float4 v = *reinterpret_cast<const float4*>(srow + c);
        const bf16x4_t b = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
        if (dst_dt == BF16) *reinterpret_cast<bf16x4_t*>(reinterpret_cast<__bf16*>(dst) + dr * ld_dst + c) = b;
        else *reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + dr * ld_dst + c) = v;
        if (dst2) *reinterpret_cast<bf16x4_t*>(dst2 + dr * ld_dst2 + c) = b;
      } else {
        for (int u = 0; u < 4 && c + u < cols; ++u) {
          const float v = srow[c + u];
          if (dst_dt == BF16) reinterpret_cast<__bf16*>(dst)[dr * ld_dst + c + u] = (__bf16)v;
          else reinterpret_cast<float*>(dst)[dr * ld_dst + c + u] = v;
          if (dst2) dst2[dr * ld_dst2 + c + u] = (__bf16)v;
        }
      }
    }
  }
}

// dst[r][j] = src[r][idx[j]] (float32 or bf16 dst) and, when dst2 is given, dst2[r][j] = bf16 of it. Four consecutive
// output columns per thread (four reads near each other: the indices ascend) and, with vec (pitches multiples of 4,
// bases aligned), one 16-byte (float32) or 8-byte (bf16) store per output; several rows per workgroup.
__global__ __launch_bounds__(256) void k_gather_cols(const float* __restrict__ src, int64_t ld_src, int rows,
                                                     const int32_t* __restrict__ idx, int s, int dlim,
                                                     void* __restrict__ dst, int dst_dt, int64_t ld_dst,
                                                     __bf16* __restrict__ dst2, int64_t ld_dst2, int vec) {
  for (int r = blockIdx.y; r < rows; r += gridDim.y) {
    const float* srow = src + (int64_t)r * ld_src;
    for (int j = 4 * (blockIdx.x * blockDim.x + threadIdx.x); j < s; j += 4 * gridDim.x * blockDim.x) {
      if (vec && j + 4 <= s) {
        const int4 c = *reinterpret_cast<const int4*>(idx + j);
        const float4 v = {srow[clampi(c.x, dlim)], srow[clampi(c.y, dlim)], srow[clampi(c.z, dlim)],
                          srow[clampi(c.w, dlim)]};
        const bf16x4_t b = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
        if (dst_dt == BF16) *reinterpret_cast<bf16x4_t*>(reinterpret_cast<__bf16*>(dst) + (int64_t)r * ld_dst + j) = b;
        else *reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + (int64_t)r * ld_dst + j) = v;
        if (dst2) *reinterpret_cast<bf16x4_t*>(dst2 + (int64_t)r * ld_dst2 + j) = b;
      } else {
        for (int u = 0; u < 4 && j + u < s; ++u) {
          const float v = srow[clampi(idx[j + u], dlim)];
          if (dst_dt == BF16) reinterpret_cast<__bf16*>(dst)[(int64_t)r * ld_dst + j + u] = (__bf16)v;
          else reinterpret_cast<float*>(dst)[(int64_t)r * ld_dst + j + u] = v;
          if (dst2) dst2[(int64_t)r * ld_dst2 + j + u] = (__bf16)v;
        }
      }
    }
  }
}

__global__ void k_split3(const float* __restrict__ src, int64_t ld_src, const int32_t* __restrict__ ridx,
                         const int32_t* __restrict__ cidx, int rlim, int clim, int sub_eye, int rows, int cols, int prows,
                         int pcols, __bf16* __restrict__ dst, int64_t ld_dst, int64_t tstride, int lo_mask,
                         float* __restrict__ D, int64_t ld_d) {
  for (int i = blockIdx.y; i < prows; i += gridDim.y)
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < pcols; j += gridDim.x * blockDim.x) {
      float x = 0.f;
      const bool in = i < rows && j < cols;
      if (in) {
        const int r = ridx ? clampi(ridx[i], rlim) : i, c = cidx ? clampi(cidx[j], clim) : j;
        x = src[(int64_t)r * ld_src + c] - (sub_eye && i == j ? 1.f : 0.f);
        if (D) D[(int64_t)i * ld_d + j] = x;
      }
      const __bf16 hi = (__bf16)x, lo = (__bf16)(x - (float)hi);
      __bf16* o = dst + (int64_t)i * ld_dst + j;
#pragma unroll
      for (int t = 0; t < 3; ++t) o[t * tstride] = (lo_mask >> t) & 1 ? lo : hi;
    }
}

// dst[r][idx[j]] = src[r][j]: four consecutive source columns per thread (one 16-byte load with vec), several rows
// per workgroup.
__global__ __launch_bounds__(256) void k_scatter_cols(const float* __restrict__ src, int64_t ld_src, int rows,
                                                      const int32_t* __restrict__ idx, int s, int dlim,
                                                      void* __restrict__ dst, int dst_dt, int64_t ld_dst, int vec) {
  for (int r = blockIdx.y; r < rows; r += gridDim.y)
    for (int j = 4 * (blockIdx.x * blockDim.x + threadIdx.x); j < s; j += 4 * gridDim.x * blockDim.x) {
      float v[4];
      int c[4];
      const int nv = min(4, s - j);
      if (vec && nv == 4) {
        const float4 f = *reinterpret_cast<const float4*>(src + (int64_t)r * ld_src + j);
        const int4 q = *reinterpret_cast<const int4*>(idx + j);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        c[0] = q.x; c[1] = q.y; c[2] = q.z; c[3] = q.w;
      } else {
        for (int u = 0; u < nv; ++u) { v[u] = src[(int64_t)r * ld_src + j + u]; c[u] = idx[j + u]; }
      }
      for (int u = 0; u < nv; ++u) {
        const int64_t o = (int64_t)r * ld_dst + clampi(c[u], dlim);
        if (dst_dt == BF16) reinterpret_cast<__bf16*>(dst)[o] = (__bf16)v[u];
        else reinterpret_cast<float*>(dst)[o] = v[u];
      }
    }
}

__global__ void k_gather_rows(const void* __restrict__ src, int src_dt, int64_t ld_src, const int32_t* __restrict__ idx,
                              int s, int dlim, int cols, void* __restrict__ dst, int dst_dt, int64_t ld_dst,
                              __bf16* __restrict__ dst2, int64_t ld_dst2) {
  for (int i = blockIdx.y; i < s; i += gridDim.y) {
    const int64_t row = (int64_t)clampi(idx[i], dlim) * ld_src;
    for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < cols; c += gridDim.x * blockDim.x) {
      const float v = src_dt == BF16 ? (float)reinterpret_cast<const __bf16*>(src)[row + c]
                                     : reinterpret_cast<const float*>(src)[row + c];
      if (dst_dt == BF16) reinterpret_cast<__bf16*>(dst)[(int64_t)i * ld_dst + c] = (__bf16)v;
      else reinterpret_cast<float*>(dst)[(int64_t)i * ld_dst + c] = v;
      if (dst2) dst2[(int64_t)i * ld_dst2 + c] = (__bf16)v;
    }
  }
}

// dst[i][cidx[j]] = C[ridx[i]][j] (i < sr, j < sc), with a bf16 copy into dst2[i][cidx[j]]
__global__ void k_patch_block(const float* __restrict__ C, int64_t ldc, const int32_t* __restrict__ ridx, int rlim,
                              const int32_t* __restrict__ cidx, int clim, int sr, int sc, float* __restrict__ dst,
                              int64_t ld_dst, __bf16* __restrict__ dst2, int64_t ld_dst2) {
  for (int i = blockIdx.y; i < sr; i += gridDim.y) {
    const int64_t row = (int64_t)clampi(ridx[i], rlim) * ldc;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < sc; j += gridDim.x * blockDim.x) {
      const float v = C[row + j];
      const int c = clampi(cidx[j], clim);
      dst[(int64_t)i * ld_dst + c] = v;
      dst2[(int64_t)i * ld_dst2 + c] = (__bf16)v;
    }
  }
}

// ---- counter-based index sampler -------------------------------------------------------------------------
// SplitMix64 output step (Steele, Lea and Flood, OOPSLA 2014): advance by the golden gamma and finalize.
__host__ __device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// The rank of index i is the number of indices j with (key_j, j) < (key_i, i). Index set mode (perm null):
// flags[i] = 1 when the rank is below s. Permutation mode: perm[rank] = i and, when inv is given, inv[i] = rank (the
// ranks are a bijection onto [0, d), so every entry is written once). A workgroup of kRankWaves waves ranks 64
// indices (lane = i): each chunk of kRankChunk keys is hashed into LDS once, wave w compares against its 64-key slice
// of the chunk, and the waves' integer counts are summed at the end (the order of an integer sum does not matter).
constexpr int kRankWaves = 16, kRankChunk = kRankWaves * 64;
__global__ void __launch_bounds__(kRankChunk) k_sample_rank(int d, int s, uint64_t h, int32_t* __restrict__ flags,
                                                            int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ uint64_t kj[kRankChunk];
  __shared__ int part[kRankWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  const uint64_t ki = splitmix64(h ^ (uint64_t)(i < d ? i : 0));
  int rank = 0;
  for (int j0 = 0; j0 < d; j0 += kRankChunk) {
    const int j = j0 + threadIdx.x;
    kj[threadIdx.x] = j < d ? splitmix64(h ^ (uint64_t)j) : 0ull;
    __syncthreads();
    const int t0 = w * 64, t1 = min(t0 + 64, d - j0);
    for (int t = t0; t < t1; ++t) {
      const uint64_t kv = kj[t];
      const int jj = j0 + t;
      rank += (kv < ki) || (kv == ki && jj < i);
    }
    __syncthreads();
  }
  part[w][lane] = rank;
  __syncthreads();
  if (w == 0) {
    int r = 0;
    for (int q = 0; q < kRankWaves; ++q) r += part[q][lane];
    if (i < d) {
      if (perm) {
        perm[r] = i;
        if (inv) inv[i] = r;
      } else {
        flags[i] = r < s ? 1 : 0;
      }
    }
  }
}

// out[i][j] = in[ri][cj] with ri = row_idx[i] (or i) and cj = col_idx[j] (or j), both clamped into the source;
// E is the element type (2 or 4 bytes: the bits are moved as they are). Rows of the output over blockIdx.y (grid
// stride), columns over threads: the stores are coalesced, the reads scatter within one source row. The general
// form (long rows, row gathers); k_gather_cols_lds below takes the column gathers of activations.
template <typename E>
__global__ __launch_bounds__(256) void k_gather2d(int rows, int cols, const E* __restrict__ in, int64_t ldi, int in_rows,
                                                  int in_cols, const int32_t* __restrict__ row_idx,
                                                  const int32_t* __restrict__ col_idx, E* __restrict__ out, int64_t ldo) {
  for (int i = blockIdx.y; i < rows; i += gridDim.y) {
    const int64_t src = (int64_t)(row_idx ? clampi(row_idx[i], in_rows) : i) * ldi;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < cols; j += gridDim.x * blockDim.x)
      out[(int64_t)i * ldo + j] = in[src + (col_idx ? clampi(col_idx[j], in_cols) : j)];
  }
}

// Column gather of 2-byte elements through LDS: a workgroup keeps the (clamped) column indices in LDS and, for each
// of its rows, copies the source row into LDS with 16-byte loads, then writes 8 gathered elements per thread as one
// 16-byte store. Needs in_cols <= GC_MAX_IN and cols <= GC_MAX_OUT (LDS) and 16-byte aligned rows (base, ldi and ldo
// multiples of 8 elements); a partial last chunk of a row is read and written element by element, so nothing past
// in_cols of a source row or cols of an output row is touched.
constexpr int GC_MAX_IN = 8192, GC_MAX_OUT = 8192, GC_ROWS = 16;
__global__ __launch_bounds__(256) void k_gather_cols_lds(int rows, int cols, const uint16_t* __restrict__ in,
                                                         int64_t ldi, int in_rows, int in_cols,
                                                         const int32_t* __restrict__ row_idx,
                                                         const int32_t* __restrict__ col_idx,
                                                         uint16_t* __restrict__ out, int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t rowbuf[GC_MAX_IN];
  __shared__ int32_t cidx[GC_MAX_OUT];
  for (int j = threadIdx.x; j < cols; j += blockDim.x) cidx[j] = clampi(col_idx[j], in_cols);
  const int nch_in = (in_cols + 7) / 8, nch_out = (cols + 7) / 8;
  const int r0 = blockIdx.x * GC_ROWS, r1 = min(rows, r0 + GC_ROWS);
  for (int i = r0; i < r1; ++i) {
    const uint16_t* src = in + (int64_t)(row_idx ? clampi(row_idx[i], in_rows) : i) * ldi;
    __syncthreads();  // the previous row's gathers are done with rowbuf (and cidx is written)
    for (int q = threadIdx.x; q < nch_in; q += blockDim.x) {
      if (8 * q + 8 <= in_cols) {
        *reinterpret_cast<uint4*>(rowbuf + 8 * q) = *reinterpret_cast<const uint4*>(src + 8 * q);
      } else {
        for (int j = 8 * q; j < in_cols; ++j) rowbuf[j] = src[j];
      }
    }
    __syncthreads();
    uint16_t* dst = out + (int64_t)i * ldo;
    for (int q = threadIdx.x; q < nch_out; q += blockDim.x) {
      const int j0 = 8 * q;
      if (j0 + 8 <= cols) {
        uint16_t v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = rowbuf[cidx[j0 + t]];
        uint4 w;
        w.x = v[0] | ((uint32_t)v[1] << 16); w.y = v[2] | ((uint32_t)v[3] << 16);
        w.z = v[4] | ((uint32_t)v[5] << 16); w.w = v[6] | ((uint32_t)v[7] << 16);
        *reinterpret_cast<uint4*>(dst + j0) = w;
      } else {
        for (int j = j0; j < cols; ++j) dst[j] = rowbuf[cidx[j]];
      }
    }
  }
}

// one workgroup: stream compaction of the flagged indices in ascending order
__global__ void k_sample_compact(int d, const int32_t* __restrict__ flags, int32_t* __restrict__ idx) {
  constexpr int NT = 1024;
  __shared__ int sc[NT];
  int base = 0;
  for (int c0 = 0; c0 < d; c0 += NT) {
    const int i = c0 + threadIdx.x;
    const int f = i < d ? flags[i] : 0;
    sc[threadIdx.x] = f;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {  // inclusive Hillis-Steele scan
      const int v = threadIdx.x >= off ? sc[threadIdx.x - off] : 0;
      __syncthreads();
      sc[threadIdx.x] += v;
      __syncthreads();
    }
    if (f) idx[base + sc[threadIdx.x] - 1] = i;
    const int tot = sc[NT - 1];
    __syncthreads();
    base += tot;
  }
}

// out (bp x ldo rows per primitive, columns past bp zero) = bf16(prim - I); blockIdx.y = primitive
// four consecutive elements of a row per thread (bp and ldo multiples of 4: one 16-byte load, one 8-byte store)
__global__ void k_delta_bf16(const float* __restrict__ prim, int bp, int ldo, __bf16* __restrict__ out) {
  const int p = blockIdx.y;
  const int e = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (e >= bp * ldo) return;
  const int i = e / ldo, j = e - i * ldo;
  const float* row = prim + ((int64_t)p * bp + i) * bp;
  bf16x4_t w;
  if ((bp & 3) == 0 && (ldo & 3) == 0) {
    const float4 v = j < bp ? *reinterpret_cast<const float4*>(row + j) : float4{0.f, 0.f, 0.f, 0.f};
    const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = (__bf16)(j + u < bp ? f[u] - (i == j + u ? 1.f : 0.f) : 0.f);
    *reinterpret_cast<bf16x4_t*>(out + (int64_t)p * bp * ldo + e) = w;
  } else {
    for (int u = 0; u < 4 && e + u < bp * ldo; ++u) {
      const int ii = (e + u) / ldo, jj = (e + u) - ii * ldo;
      const float v = jj < bp ? prim[((int64_t)p * bp + ii) * bp + jj] - (ii == jj ? 1.f : 0.f) : 0.f;
      out[(int64_t)p * bp * ldo + e + u] = (__bf16)v;
    }
  }
}

__device__ __forceinline__ float ld_dt(const void* p, int dt, int64_t i) {
  return dt == BF16 ? (float)reinterpret_cast<const __bf16*>(p)[i] : reinterpret_cast<const float*>(p)[i];
}

// The stacked coefficient matrices C_0..C_k of primitive p = blockIdx.y of side blockIdx.z (see launch_adjoint_coefs),
// each stored ldp x ldp (rows and columns past bp zero). Thread x covers VEC consecutive elements (r, c0..c0+VEC) of
// every C_j: it reads the k saved powers at those elements once (powers are bp x ldp blocks) and writes the k + 1
// coefficient blocks from registers. KMAX bounds k (unrolled, so the powers stay in registers).
template <typename T, int VEC, int KMAX>
__global__ void k_adjoint_coefs(const CoefGroup G) {
  CoefSide sd;
  {
    const CoefSide& t = G.s[blockIdx.z];
    sd.powers = keep_s(t.powers); sd.out = keep_s(t.out); sd.nprim = keep_s(t.nprim);
  }
  const int nprim = sd.nprim, bp = G.bp, ldp = G.ldp, k = G.k;
  const int p = blockIdx.y;
  if (p >= nprim) return;
  const T* __restrict__ powers = reinterpret_cast<const T*>(sd.powers);
  T* __restrict__ out = reinterpret_cast<T*>(sd.out);
  const int pq = ldp * ldp;
  const int rc0 = (blockIdx.x * blockDim.x + threadIdx.x) * VEC;
  if (rc0 >= pq) return;
  const int r = rc0 / ldp, c0 = rc0 - r * ldp;  // VEC divides ldp: the VEC elements share the row
  float q[KMAX][VEC];  // q[t-1] = Q^t at this thread's elements
#pragma unroll
  for (int t = 1; t <= KMAX; ++t) {
#pragma unroll
    for (int u = 0; u < VEC; ++u) q[t - 1][u] = 0.f;
    if (t <= k && r < bp) {
      const T* src = powers + ((size_t)(t - 1) * nprim + p) * bp * ldp + (size_t)r * ldp + c0;
      if (c0 + VEC <= bp) {  // whole group inside the block: one VEC-wide load (the launcher checked the alignment)
        T w[VEC];
        __builtin_memcpy(w, __builtin_assume_aligned(src, sizeof(T) * VEC), sizeof(w));
#pragma unroll
        for (int u = 0; u < VEC; ++u) q[t - 1][u] = (float)w[u];
      } else {
#pragma unroll
        for (int u = 0; u < VEC; ++u)
          if (c0 + u < bp) q[t - 1][u] = (float)src[u];
      }
    }
  }
  // C_j = [j > 0] a_{j+1} (-1)^j I + sum_{t=1}^{k-j} a_{t+j+1} (-1)^{t+j} Q^t, with a_i = 2 (i <= k), a_{k+1} = 1
#pragma unroll
  for (int j = 0; j <= KMAX; ++j) {
    if (j > k) break;
    float v[VEC];
#pragma unroll
    for (int u = 0; u < VEC; ++u) v[u] = 0.f;
    if (r < bp) {
      if (j > 0) {
        const float a = (j + 1 <= k ? 2.f : 1.f) * ((j & 1) ? -1.f : 1.f);
#pragma unroll
        for (int u = 0; u < VEC; ++u)
          if (c0 + u == r) v[u] = a;
      }
#pragma unroll
      for (int t = 1; t <= KMAX; ++t) {
        if (t > k - j) break;
        const int i = t + j + 1;
        const float a = (i <= k ? 2.f : 1.f) * (((t + j) & 1) ? -1.f : 1.f);
#pragma unroll
        for (int u = 0; u < VEC; ++u) v[u] += a * q[t - 1][u];
      }
    }
    T* dst = out + ((size_t)p * (k + 1) + j) * pq + rc0;
    T w[VEC];
#pragma unroll
    for (int u = 0; u < VEC; ++u) w[u] = (T)v[u];
    __builtin_memcpy(__builtin_assume_aligned(dst, sizeof(T) * VEC), w, sizeof(w));
  }
}

// prim = I + 2 Q + 2 (P_2 + ... + P_k) + P_{k+1}, where prim holds P_{k+1} on entry, Q comes from theta
// (float32, exact) and P_t = powers[t-1] (dtype dt); k >= 1. Side blockIdx.z, primitive blockIdx.y, tile pair
// blockIdx.x (the same tiling as k_theta_prep). A thread takes V consecutive columns of a row (32 / V threads per
// tile row), so the powers, prim and q2 move as V-element loads and stores where the row holds them; every
// element's sum is formed in the same order as one element at a time.
template <int V>
__global__ __launch_bounds__(256) void k_chain_finalize(const FinGroup G) {
  __shared__ float tr[32][33];
  FinSide a;
  {
    const FinSide& t = G.s[blockIdx.z];
    a.theta = keep_s(t.theta); a.powers = keep_s(t.powers); a.prim = keep_s(t.prim); a.mode = keep_s(t.mode);
    a.d = keep_s(t.d); a.bp = keep_s(t.bp); a.nprim = keep_s(t.nprim); a.k = keep_s(t.k); a.dt = keep_s(t.dt);
    a.ldp = keep_s(t.ldp); a.q2 = keep_s(t.q2);
  }
  const int bp = a.bp, p = blockIdx.y, nt = (bp + 31) / 32;
  if (p >= a.nprim || (int)blockIdx.x >= nt * (nt + 1) / 2) return;
  int ti, tj;
  tile_pair_of(blockIdx.x, bp, ti, tj);
  const int c = prim_size(a.mode, a.d, bp, p);
  float up[4], lo[4];
  q_tile_pair(a.theta, theta_off(bp, p), c, ti, tj, tr, up, lo);  // stages the upper tile in tr
  constexpr int TPR = 32 / V, RPP = 256 / TPR;
  const int cv = (threadIdx.x % TPR) * V, r0 = threadIdx.x / TPR;
  const bool diag = ti == tj;
  float* prim = a.prim + (int64_t)p * bp * bp;
  const float* q2 = a.q2 ? a.q2 + (int64_t)p * bp * bp : nullptr;
  for (int h = 0; h < 2; ++h) {
    if (h == 1 && diag) break;
    const int ri = h ? tj : ti, cj = h ? ti : tj;
    for (int r = r0; r < 32; r += RPP) {
      const int i = ri * 32 + r, j0 = cj * 32 + cv;
      if (i >= bp || j0 >= bp) continue;
      const int64_t e0 = (int64_t)i * bp + j0;
      if (j0 + V <= bp) {
        float s2[V], x[V], v[V], pv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) s2[e] = 0.f;
        for (int t = a.q2 ? 3 : 2; t <= a.k; ++t) {
          ld_row<V>(a.powers, a.dt, (((int64_t)(t - 1) * a.nprim + p) * bp + i) * a.ldp + j0, x);
#pragma unroll
          for (int e = 0; e < V; ++e) s2[e] += x[e];
        }
        ld_row<V>(prim, F32, e0, pv);
        if (q2) ld_row<V>(q2, F32, e0, x);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          v[e] = (i == j0 + e ? 1.f : 0.f) + 2.f * q_of(tr, h, diag, r, cv + e) + 2.f * s2[e];
          if (q2) {
            v[e] += (a.k >= 2 ? 0.5f : 0.25f) * x[e];
            if (a.k >= 2) v[e] += pv[e];
          } else {
            v[e] += pv[e];
          }
        }
        st_row<V>(prim, F32, e0, v);
      } else {  // the last columns of a ragged block, one at a time
        for (int e = 0; e < V && j0 + e < bp; ++e) {
          const int j = j0 + e;
          float s2 = 0.f;
          for (int t = a.q2 ? 3 : 2; t <= a.k; ++t)
            s2 += ld_dt(a.powers, a.dt, (((int64_t)(t - 1) * a.nprim + p) * bp + i) * a.ldp + j);
          float v = (i == j ? 1.f : 0.f) + 2.f * q_of(tr, h, diag, r, cv + e) + 2.f * s2;
          if (q2) {
            v += (a.k >= 2 ? 0.5f : 0.25f) * q2[e0 + e];
            if (a.k >= 2) v += prim[e0 + e];
          } else {
            v += prim[e0 + e];
          }
          prim[e0 + e] = v;
        }
      }
    }
  }
}


}  // namespace

hipError_t launch_chain_finalize_group(const FinGroup& g, hipStream_t st) {
  if (g.n <= 0) return hipSuccess;
  if (g.n > MAXG) return hipErrorInvalidValue;
  int64_t most = 0;
  double bytes = 0;
  for (int i = 0; i < g.n; ++i) {
    const FinSide& a = g.s[i];
    const int64_t total = (int64_t)a.nprim * a.bp * a.bp;
    most = std::max(most, total);
    bytes += (double)total * (8 + 4 + (a.k - 1) * dtype_size(a.dt) + (a.q2 ? 4 : 0));
  }
  if (most == 0) return hipSuccess;
  int bp = 0, ny = 0;
  for (int i = 0; i < g.n; ++i) { bp = std::max(bp, g.s[i].bp); ny = std::max(ny, g.s[i].nprim); }
  if (ny > 65535) return hipErrorInvalidValue;
  const int nt = (bp + 31) / 32;
  // V: the widest of 4, 2, 1 consecutive elements that every side's rows hold at aligned addresses
  auto fits = [&](int V) {
    for (int i = 0; i < g.n; ++i) {
      const FinSide& a = g.s[i];
      if (a.bp % V || a.ldp % V) return false;
      if (reinterpret_cast<uintptr_t>(a.prim) % (4 * V) || reinterpret_cast<uintptr_t>(a.q2) % (4 * V) ||
          reinterpret_cast<uintptr_t>(a.powers) % (dtype_size(a.dt) * V))
        return false;
    }
    return true;
  };
  ProfScope prof(7, st, 0, bytes);
  const dim3 grid(nt * (nt + 1) / 2, ny, g.n);
  if (fits(4)) hipLaunchKernelGGL(k_chain_finalize<4>, grid, dim3(kThreads), 0, st, g);
  else if (fits(2)) hipLaunchKernelGGL(k_chain_finalize<2>, grid, dim3(kThreads), 0, st, g);
  else hipLaunchKernelGGL(k_chain_finalize<1>, grid, dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_chain_finalize(const float* theta, int mode, int d, int bp, int nprim, int k, const void* powers,
                                 int dt, int ldp, float* prim, hipStream_t st, const float* q2) {
  FinGroup g;
  g.n = 1;
  FinSide& a = g.s[0];
  a.q2 = q2;
  a.theta = theta; a.powers = powers; a.prim = prim; a.mode = mode; a.d = d; a.bp = bp; a.nprim = nprim; a.k = k;
  a.dt = dt; a.ldp = ldp;
  return launch_chain_finalize_group(g, st);
}

hipError_t launch_delta_bf16(const float* prim, int nprim, int bp, int ldo, __bf16* out, hipStream_t st) {
  if (nprim <= 0 || bp <= 0) return hipSuccess;
  if (nprim > 65535 || (int64_t)bp * ldo > (1 << 30)) return hipErrorInvalidValue;
  ProfScope prof(7, st, 0, (double)nprim * bp * (4.0 * bp + 2.0 * ldo));
  const dim3 grid((bp * ldo / 4 + kThreads) / kThreads, nprim);
  hipLaunchKernelGGL(k_delta_bf16, grid, dim3(kThreads), 0, st, prim, bp, ldo, out);
  return hipGetLastError();
}

hipError_t launch_adjoint_coefs_group(const CoefGroup& g, int dt, hipStream_t st) {
  if (g.n <= 0) return hipSuccess;
  if (g.n > MAXG) return hipErrorInvalidValue;
  const int ldp = g.ldp, k = g.k, pq = ldp * ldp;
  if (k < 1 || k > 16) return hipErrorInvalidValue;
  int ny = 0;
  double total = 0;
  for (int i = 0; i < g.n; ++i) {
    ny = std::max(ny, g.s[i].nprim);
    total += (double)g.s[i].nprim * pq;
  }
  if (total == 0) return hipSuccess;
  if ((int64_t)ldp * ldp > (1 << 30) || ny > 65535) return hipErrorInvalidValue;
  ProfScope prof(7, st, 0, total * dtype_size(dt) * (2 * k + 1));
#define POET_COEF(T_, V_, KM_)                                                                          \
  hipLaunchKernelGGL((k_adjoint_coefs<T_, V_, KM_>), dim3((pq / V_ + kThreads - 1) / kThreads, ny, g.n), \
                     dim3(kThreads), 0, st, g)
  // VEC elements of a row per thread, moved as one load / store: VEC divides ldp and every side's powers and
  // output are aligned to VEC elements
  uintptr_t bits = 0;
  for (int i = 0; i < g.n; ++i)
    bits |= reinterpret_cast<uintptr_t>(g.s[i].powers) | reinterpret_cast<uintptr_t>(g.s[i].out);
  const bool a16 = (bits & 15) == 0, a8 = (bits & 7) == 0;
  if (dt == BF16 && ldp % 8 == 0 && a16) {
    if (k <= 8) POET_COEF(__bf16, 8, 8);
    else POET_COEF(__bf16, 8, 16);
  } else if (dt == BF16 && ldp % 4 == 0 && a8) {
    if (k <= 8) POET_COEF(__bf16, 4, 8);
    else POET_COEF(__bf16, 4, 16);
  } else if (dt == BF16) {
    if (k <= 8) POET_COEF(__bf16, 1, 8);
    else POET_COEF(__bf16, 1, 16);
  } else if (ldp % 4 == 0 && a16) {
    if (k <= 8) POET_COEF(float, 4, 8);
    else POET_COEF(float, 4, 16);
  } else {
    if (k <= 8) POET_COEF(float, 1, 8);
    else POET_COEF(float, 1, 16);
  }
#undef POET_COEF
  return hipGetLastError();
}

hipError_t launch_adjoint_coefs(const void* powers, int dt, int nprim, int bp, int ldp, int k, void* out, hipStream_t st) {
  CoefGroup g;
  g.n = 1; g.bp = bp; g.ldp = ldp; g.k = k;
  g.s[0].powers = powers; g.s[0].out = out; g.s[0].nprim = nprim;
  return launch_adjoint_coefs_group(g, dt, st);
}

hipError_t launch_theta_prep_group(const PrepGroup& g, hipStream_t st) {
  if (g.n <= 0) return hipSuccess;
  if (g.n > MAXG) return hipErrorInvalidValue;
  size_t most = 0;
  double bytes = 0;
  for (int i = 0; i < g.n; ++i) {
    const PrepSide& a = g.s[i];
    const size_t total = (size_t)a.nprim * a.bp * a.bp;
    most = std::max(most, total);
    bytes += (double)total * (4 + 4 + (a.q ? dtype_size(a.q_dt) : 0));
  }
  if (most == 0) return hipSuccess;
  int bp = 0, ny = 0;
  for (int i = 0; i < g.n; ++i) { bp = std::max(bp, g.s[i].bp); ny = std::max(ny, g.s[i].nprim); }
  if (ny > 65535) return hipErrorInvalidValue;
  const int nt = (bp + 31) / 32;
  auto fits = [&](int V) {  // as in launch_chain_finalize_group
    for (int i = 0; i < g.n; ++i) {
      const PrepSide& a = g.s[i];
      if (a.bp % V || (a.q && a.ldq % V)) return false;
      if (reinterpret_cast<uintptr_t>(a.prim) % (4 * V) || reinterpret_cast<uintptr_t>(a.q) % (dtype_size(a.q_dt) * V))
        return false;
    }
    return true;
  };
  ProfScope prof(7, st, 0, bytes);
  const dim3 grid(nt * (nt + 1) / 2, ny, g.n);
  if (fits(4)) hipLaunchKernelGGL(k_theta_prep<4>, grid, dim3(kThreads), 0, st, g);
  else if (fits(2)) hipLaunchKernelGGL(k_theta_prep<2>, grid, dim3(kThreads), 0, st, g);
  else hipLaunchKernelGGL(k_theta_prep<1>, grid, dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_theta_prep(const float* theta, int mode, int d, int bp, int nprim, int k, float* prim, void* q_out,
                             int q_dt, int ldq, hipStream_t st) {
  PrepGroup g;
  g.n = 1;
  PrepSide& a = g.s[0];
  a.theta = theta; a.prim = prim; a.q = q_out; a.q_dt = q_dt; a.ldq = ldq;
  a.mode = mode; a.d = d; a.bp = bp; a.nprim = nprim; a.coef = k == 0 ? 1.f : 2.f;
  return launch_theta_prep_group(g, st);
}

hipError_t launch_qnorm(const float* theta, int mode, int d, int bp, int nprim, float* qnorm, hipStream_t st) {
  ProfScope prof(7, st, 0, (double)nprim * bp * (bp - 1) * 2.0);
  hipLaunchKernelGGL(k_qnorm, dim3(nprim), dim3(kThreads), 0, st, theta, mode, d, bp, qnorm);
  return hipGetLastError();
}

hipError_t launch_skew_project(const float* dQ, const float* G1, int mode, int d, int bp, int nprim, float* dtheta,
                               hipStream_t st) {
  const size_t total = (size_t)nprim * bp * bp;
  ProfScope prof(7, st, 0, (double)total * (G1 ? 8 : 4) + (double)total * 2);
  hipLaunchKernelGGL(k_skew_project, dim3(grid_for(total)), dim3(kThreads), 0, st, dQ, G1, mode, d, bp, nprim, dtheta);
  return hipGetLastError();
}

hipError_t launch_reduce_skew_group(const SkewGroup& g, int nsplit, hipStream_t st) {
  if (g.n <= 0) return hipSuccess;
  if (g.n > MAXG) return hipErrorInvalidValue;
  const int bp = g.bp;
  int ny = 0;
  double blocks = 0;
  for (int i = 0; i < g.n; ++i) {
    ny = std::max(ny, g.s[i].nprim);
    blocks += g.s[i].nprim;
  }
  if (ny == 0) return hipSuccess;
  if (ny > 65535 || (int64_t)bp * bp > (1 << 30)) return hipErrorInvalidValue;
  ProfScope prof(7, st, 0, blocks * bp * bp * 4.0 * (nsplit + 1) + blocks * bp * (bp - 1) * 2.0);
  const int nt = (bp + 31) / 32;
  const dim3 grid(nt * (nt + 1) / 2, ny, g.n);
  switch (nsplit) {
#define POET_RS(NS) \
  case NS: hipLaunchKernelGGL(k_reduce_skew<NS>, grid, dim3(kThreads), 0, st, g); break;
    POET_RS(1) POET_RS(2) POET_RS(4) POET_RS(8) POET_RS(16)
#undef POET_RS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_reduce_skew(const float* part, int nsplit, int64_t split_stride, const float* D, float beta, int mode,
                              int d, int bp, int nprim, float* dtheta, hipStream_t st) {
  if (nprim <= 0) return hipSuccess;
  SkewGroup g;
  g.n = 1; g.part = part; g.split_stride = split_stride; g.beta = beta; g.bp = bp;
  SkewSide& a = g.s[0];
  a.D = D; a.dtheta = dtheta; a.mode = mode; a.d = d; a.nprim = nprim; a.boff = 0;
  return launch_reduce_skew_group(g, nsplit, st);
}

// Diagonal blocks of super-block products: super-block u (size sb = g bp, row pitch sb) holds the products of
// blocks u g .. u g + g - 1; block p = u g + i is its diagonal sub-block i, copied to prim[p] (bp x bp; the extent
// past a ragged last block's size c is zero).
__global__ void k_extract_diag(const float* __restrict__ sup, int sb, int g, int bp, int d, int nprim,
                               float* __restrict__ prim) {
  const int64_t total = (int64_t)nprim * bp * bp;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(e / ((int64_t)bp * bp)), rem = (int)(e % ((int64_t)bp * bp));
    const int r = rem / bp, c = rem % bp;
    const int u = p / g, i = p % g;
    const int cp = min(bp, d - p * bp);
    prim[e] = (r < cp && c < cp) ? sup[(int64_t)u * sb * sb + (int64_t)(i * bp + r) * sb + i * bp + c] : 0.f;
  }
}

hipError_t launch_extract_diag(const float* sup, int sb, int g, int bp, int d, int nprim, float* prim, hipStream_t st) {
  const size_t n = (size_t)nprim * bp * bp;
  if (n == 0) return hipSuccess;
  ProfScope prof(7, st, 0, (double)n * 8);
  hipLaunchKernelGGL(k_extract_diag, dim3(grid_for(n)), dim3(kThreads), 0, st, sup, sb, g, bp, d, nprim, prim);
  return hipGetLastError();
}

// zero the gap columns [bp, ldp) of the nblk side-by-side blocks (block j at column j ldp) of rows rows of a bf16
// matrix with row pitch ld
__global__ void k_zero_gaps(__bf16* __restrict__ H, int64_t rows, int64_t ld, int ldp, int bp, int nblk) {
  const int gw = ldp - bp;
  const int64_t n = rows * nblk * gw;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / (nblk * gw);
    const int rem = (int)(e % (nblk * gw)), j = rem / gw, gcol = rem % gw;
    H[r * ld + (int64_t)j * ldp + bp + gcol] = (__bf16)0.f;
  }
}

hipError_t launch_zero_gaps(__bf16* H, int64_t rows, int64_t ld, int ldp, int bp, int nblk, hipStream_t st) {
  const size_t n = (size_t)rows * nblk * (ldp - bp);
  if (n == 0) return hipSuccess;
  ProfScope prof(7, st, 0, (double)n * 2);
  hipLaunchKernelGGL(k_zero_gaps, dim3(grid_for(n)), dim3(kThreads), 0, st, H, rows, ld, ldp, bp, nblk);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, size_t n, float v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  ProfScope prof(7, st, 0, (double)n * 4);
  hipLaunchKernelGGL(k_fill, dim3(grid_for(n)), dim3(kThreads), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_group(const FillGroup& g, float v, hipStream_t st) {
  size_t mx = 0, tot = 0;
  for (int i = 0; i < g.n; ++i) { mx = std::max(mx, g.a[i].n); tot += g.a[i].n; }
  if (mx == 0) return hipSuccess;
  ProfScope prof(7, st, 0, (double)tot * 4);
  hipLaunchKernelGGL(k_fill_group, dim3(std::min<unsigned>(grid_for(mx), 256), g.n), dim3(kThreads), 0, st, g, v);
  return hipGetLastError();
}

// (column blocks, rows): at most 1024 row slots, so that a workgroup of a tall copy takes several rows
static dim3 row_grid(int cols, int rows) { return dim3((cols + kThreads - 1) / kThreads, rows < 1024 ? rows : 1024); }

static bool al16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static hipError_t launch_rows4(const float* src, int64_t ld_src, const int32_t* sidx, const int32_t* didx, int dlim,
                               int rows, int cols, void* dst, int dst_dt, int64_t ld_dst, __bf16* dst2, int64_t ld_dst2,
                               hipStream_t st) {
  const bool vec = ld_src % 4 == 0 && ld_dst % 4 == 0 && (!dst2 || ld_dst2 % 4 == 0) && al16(src) &&
                   (dst_dt == BF16 ? (reinterpret_cast<uintptr_t>(dst) & 7) == 0 : al16(dst)) &&
                   (reinterpret_cast<uintptr_t>(dst2) & 7) == 0;
  hipLaunchKernelGGL(k_rows4, row_grid((cols + 3) / 4, rows), dim3(kThreads), 0, st, src, ld_src, sidx, didx, dlim, rows,
                     cols, dst, dst_dt, ld_dst, dst2, ld_dst2, vec ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_convert(const float* src, int64_t ld_src, void* dst, int64_t ld_dst, int dst_dt, int rows, int cols,
                          hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  ProfScope prof(7, st, 0, (double)rows * cols * (4 + dtype_size(dst_dt)));
  return launch_rows4(src, ld_src, nullptr, nullptr, rows, rows, cols, dst, dst_dt, ld_dst, nullptr, 0, st);
}

hipError_t launch_gather_cols_to(const float* src, int64_t ld_src, int rows, const int32_t* idx, int s, int dlim,
                                 void* dst, int dst_dt, int64_t ld_dst, hipStream_t st, __bf16* dst2, int64_t ld_dst2) {
  if (rows <= 0 || s <= 0) return hipSuccess;
  ProfScope prof(POET_K_GATHER, st, 0, (double)rows * s * (4 + dtype_size(dst_dt) + (dst2 ? 2 : 0)));
  const bool vec = ld_dst % 4 == 0 && (!dst2 || ld_dst2 % 4 == 0) && al16(idx) &&
                   (dst_dt == BF16 ? (reinterpret_cast<uintptr_t>(dst) & 7) == 0 : al16(dst)) &&
                   (reinterpret_cast<uintptr_t>(dst2) & 7) == 0;
  hipLaunchKernelGGL(k_gather_cols, row_grid((s + 3) / 4, rows), dim3(kThreads), 0, st, src, ld_src, rows, idx, s, dlim,
                     dst, dst_dt, ld_dst, dst2, ld_dst2, vec ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_gather_cols(const float* src, int64_t ld_src, int rows, const int32_t* idx, int s, int dlim, float* dst,
                              int64_t ld_dst, hipStream_t st) {
  return launch_gather_cols_to(src, ld_src, rows, idx, s, dlim, dst, F32, ld_dst, st);
}

hipError_t launch_split3(const float* src, int64_t ld_src, const int32_t* ridx, const int32_t* cidx, int rlim, int clim,
                         int sub_eye, int rows, int cols, int prows, int pcols, __bf16* dst, int64_t ld_dst,
                         int64_t tstride, int lo_mask, float* D, int64_t ld_d, hipStream_t st) {
  if (prows <= 0 || pcols <= 0) return hipSuccess;
  ProfScope prof(7, st, 0, (double)rows * cols * (D ? 8 : 4) + 6.0 * prows * pcols);
  hipLaunchKernelGGL(k_split3, row_grid(pcols, prows), dim3(kThreads), 0, st, src, ld_src, ridx, cidx, rlim, clim,
                     sub_eye, rows, cols, prows, pcols, dst, ld_dst, tstride, lo_mask, D, ld_d);
  return hipGetLastError();
}

hipError_t launch_scatter_cols_to(const float* src, int64_t ld_src, int rows, const int32_t* idx, int s, int dlim,
                                  void* dst, int dst_dt, int64_t ld_dst, hipStream_t st) {
  if (rows <= 0 || s <= 0) return hipSuccess;
  ProfScope prof(POET_K_GATHER, st, 0, (double)rows * s * (4 + dtype_size(dst_dt)));
  const bool vec = ld_src % 4 == 0 && al16(src) && al16(idx);
  hipLaunchKernelGGL(k_scatter_cols, row_grid((s + 3) / 4, rows), dim3(kThreads), 0, st, src, ld_src, rows, idx, s, dlim,
                     dst, dst_dt, ld_dst, vec ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_patch_block(const float* C, int64_t ldc, const int32_t* ridx, int rlim, const int32_t* cidx, int clim,
                              int sr, int sc, float* dst, int64_t ld_dst, __bf16* dst2, int64_t ld_dst2, hipStream_t st) {
  if (sr <= 0 || sc <= 0) return hipSuccess;
  ProfScope prof(POET_K_GATHER, st, 0, (double)sr * sc * 10);
  hipLaunchKernelGGL(k_patch_block, row_grid(sc, sr), dim3(kThreads), 0, st, C, ldc, ridx, rlim, cidx, clim, sr, sc, dst,
                     ld_dst, dst2, ld_dst2);
  return hipGetLastError();
}

hipError_t launch_scatter_cols(const float* src, int64_t ld_src, int rows, const int32_t* idx, int s, int dlim,
                               float* dst, int64_t ld_dst, hipStream_t st) {
  return launch_scatter_cols_to(src, ld_src, rows, idx, s, dlim, dst, F32, ld_dst, st);
}

hipError_t launch_gather_rows_to(const void* src, int src_dt, int64_t ld_src, const int32_t* idx, int s, int dlim,
                                 int cols, void* dst, int dst_dt, int64_t ld_dst, hipStream_t st, __bf16* dst2,
                                 int64_t ld_dst2) {
  if (s <= 0 || cols <= 0) return hipSuccess;
  ProfScope prof(POET_K_GATHER, st, 0, (double)s * cols * (dtype_size(dst_dt) + dtype_size(src_dt) + (dst2 ? 2 : 0)));
  if (src_dt == F32)
    return launch_rows4(reinterpret_cast<const float*>(src), ld_src, idx, nullptr, dlim, s, cols, dst, dst_dt, ld_dst,
                        dst2, ld_dst2, st);
  hipLaunchKernelGGL(k_gather_rows, row_grid(cols, s), dim3(kThreads), 0, st, src, src_dt, ld_src, idx, s, dlim, cols,
                     dst, dst_dt, ld_dst, dst2, ld_dst2);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, int src_dt, int64_t ld_src, const int32_t* idx, int s, int dlim, int cols,
                              float* dst, int64_t ld_dst, hipStream_t st) {
  return launch_gather_rows_to(src, src_dt, ld_src, idx, s, dlim, cols, dst, F32, ld_dst, st);
}

hipError_t launch_scatter_rows(const float* src, int64_t ld_src, const int32_t* idx, int s, int dlim, int cols, void* dst,
                               int dst_dt, int64_t ld_dst, hipStream_t st) {
  if (s <= 0 || cols <= 0) return hipSuccess;
  ProfScope prof(POET_K_GATHER, st, 0, (double)s * cols * (4 + dtype_size(dst_dt)));
  return launch_rows4(src, ld_src, nullptr, idx, dlim, s, cols, dst, dst_dt, ld_dst, nullptr, 0, st);
}

uint64_t sampler_hash(uint64_t seed, uint32_t linear_id, uint32_t side, uint32_t epoch) {
  uint64_t h = splitmix64(seed);
  h = splitmix64(h ^ (uint64_t)linear_id);
  h = splitmix64(h ^ (uint64_t)side);
  return splitmix64(h ^ (uint64_t)epoch);
}

hipError_t launch_sample(int d, int s, uint64_t h, int32_t* flags, int32_t* idx, hipStream_t st) {
  if (d <= 0 || s <= 0) return hipSuccess;
  ProfScope prof(7, st, 0, (double)d * 4 + (double)s * 4);
  hipLaunchKernelGGL(k_sample_rank, dim3((d + 63) / 64), dim3(kRankChunk), 0, st, d, s, h, flags, nullptr, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sample_compact, dim3(1), dim3(1024), 0, st, d, flags, idx);
  return hipGetLastError();
}

hipError_t launch_sample_permutation(int d, uint64_t h, int32_t* perm, int32_t* inv, hipStream_t st) {
  if (d <= 0) return hipSuccess;
  ProfScope prof(POET_K_GATHER, st, 0, (double)d * 8);
  hipLaunchKernelGGL(k_sample_rank, dim3((d + 63) / 64), dim3(kRankChunk), 0, st, d, 0, h, nullptr, perm, inv);
  return hipGetLastError();
}

hipError_t launch_gather2d(int rows, int cols, int elem_bytes, const void* in, int64_t ldi, int in_rows, int in_cols,
                           const int32_t* row_idx, const int32_t* col_idx, void* out, int64_t ldo, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  ProfScope prof(POET_K_GATHER, st, 0, 2.0 * elem_bytes * (double)rows * cols);
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (elem_bytes == 2 && col_idx && in_cols <= GC_MAX_IN && cols <= GC_MAX_OUT && ldi % 8 == 0 && ldo % 8 == 0 &&
      a16(in) && a16(out)) {
    hipLaunchKernelGGL(k_gather_cols_lds, dim3((rows + GC_ROWS - 1) / GC_ROWS), dim3(256), 0, st, rows, cols,
                       reinterpret_cast<const uint16_t*>(in), ldi, in_rows, in_cols, row_idx, col_idx,
                       reinterpret_cast<uint16_t*>(out), ldo);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)std::min(65535, (cols + 255) / 256), (unsigned)std::min(rows, 65535));
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_gather2d<uint16_t>, grid, dim3(256), 0, st, rows, cols, reinterpret_cast<const uint16_t*>(in),
                       ldi, in_rows, in_cols, row_idx, col_idx, reinterpret_cast<uint16_t*>(out), ldo);
  else
    hipLaunchKernelGGL(k_gather2d<uint32_t>, grid, dim3(256), 0, st, rows, cols, reinterpret_cast<const uint32_t*>(in),
                       ldi, in_rows, in_cols, row_idx, col_idx, reinterpret_cast<uint32_t*>(out), ldo);
  return hipGetLastError();
}

}  // namespace poet

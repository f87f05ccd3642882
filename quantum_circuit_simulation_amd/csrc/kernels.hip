// gfx950 kernels for tree contraction: complex64 data on FP32 arithmetic
// (FP32 MFMA), complex128 data on FP64 arithmetic (FP64 MFMA).
//
// Every pairwise step of the page "Parallelizing Large-Scale Tensor Network
// Contraction on Multiple GPUs" (section 1.1) is, after lifetime ordering
// (section 1.4), C[i, j] = sum_l X[i, l] * Y[j, l] with both operands stored
// K-innermost.  Kernels by step shape:
//   k_cgemm, k_cgemm_tile - MFMA tiles (v_mfma_f32_32x32x2_f32) for steps
//               with both sides > 16: persistent workgroups for short K
//               chunks, one tile per workgroup for long ones; the complex
//               product is a real GEMM whose K axis carries (re, im);
//   k_zgemm   - the same on v_mfma_f64_16x16x4_f64 for complex128;
//   k_skinny_flat, k_skinny_small, k_skinny_rows, k_skinny, k_skinny_z -
//               VALU streaming for steps with one side <= 16 (HBM-bound);
//   k_tiny    - one workgroup per step for the many small early-tree steps,
//               a whole launch group per launch;
//   k_split_reduce - sums split-K partials into C.
// Outputs are stored through "runs": rowoff(i) + coloff(j), so a product
// whose order interleaves the two operands' modes is written in place with
// no separate permute.  k_copy_tiled / k_copy are strided permutes used only
// for leaf staging and for the naive-order ablation; k_header fills the
// workspace's pointer table and descriptor blob.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <type_traits>

#include "kernels.hpp"

namespace tnc {

// Name of the last kernel a launcher enqueued on this thread (for the timed
// executor's per-launch report).
thread_local char g_kernel_name[64];

const char *last_kernel_name() { return g_kernel_name; }
void clear_kernel_name() { g_kernel_name[0] = 0; }

namespace {

void note_kernel(const char *name) { std::snprintf(g_kernel_name, sizeof(g_kernel_name), "%s", name); }
template <typename... A>
void note_kernel(const char *fmt, A... args) {
  std::snprintf(g_kernel_name, sizeof(g_kernel_name), fmt, args...);
}
void note_append(const char *what) {
  size_t n = std::strlen(g_kernel_name);
  std::snprintf(g_kernel_name + n, sizeof(g_kernel_name) - n, "%s", what);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void cmac(float2 &acc, float2 a, float2 b) {
  acc.x = fmaf(a.x, b.x, acc.x);
  acc.x = fmaf(-a.y, b.y, acc.x);
  acc.y = fmaf(a.x, b.y, acc.y);
  acc.y = fmaf(a.y, b.x, acc.y);
}

__device__ __forceinline__ void cmac(double2 &acc, double2 a, double2 b) {
  acc.x = fma(a.x, b.x, acc.x);
  acc.x = fma(-a.y, b.y, acc.x);
  acc.y = fma(a.x, b.y, acc.y);
  acc.y = fma(a.y, b.x, acc.y);
}

template <typename T>
__device__ __forceinline__ T czero() {
  T z;
  z.x = 0;
  z.y = 0;
  return z;
}

// Offset in C (entries) of index `idx` along one side, runs outermost first.
// Indices below 2^32 (every run size then fits too) take 32-bit division, or
// a shift and a mask for a run size that is a power of two (every run of a
// network whose modes have extent 2).
__device__ __forceinline__ int64_t run_offset(int64_t idx, const RunDev *r, int n) {
  int64_t off = 0;
  if (idx < (int64_t(1) << 32)) {
    uint32_t i = (uint32_t)idx;
    for (int q = n - 1; q >= 0 && i != 0; --q) {
      const int64_t sz = r[q].size;
      if (sz >= (int64_t(1) << 32)) {
        off += (int64_t)i * r[q].stride;
        i = 0;
        break;
      }
      const uint32_t s32 = (uint32_t)sz;
      uint32_t nx, rem;
      if ((s32 & (s32 - 1u)) == 0u) {
        nx = i >> (__ffs(s32) - 1);
        rem = i & (s32 - 1u);
      } else {
        nx = i / s32;
        rem = i - nx * s32;
      }
      off += (int64_t)rem * r[q].stride;
      i = nx;
    }
    return off;
  }
  for (int q = n - 1; q >= 0; --q) {
    const int64_t sz = r[q].size;
    const int64_t d = idx % sz;
    idx /= sz;
    off += d * r[q].stride;
  }
  return off;
}

template <typename T>
__device__ __forceinline__ void store_c(T *p, T v, int beta) {
  if (beta) {
    T o = *p;
    v.x += o.x;
    v.y += o.y;
  }
  *p = v;
}

__device__ __forceinline__ bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// ---------------------------------------------------------------------------
// device pointer table

constexpr int kPtrsPerLaunch = 400;  // 3.2 KB of kernel arguments
struct PtrChunk {
  void *p[kPtrsPerLaunch];
  int32_t count;
  int32_t first;
};

// Workspace header in one launch: block 0 also writes the first pointer chunk;
// every block copies 16-byte words of the descriptor blob straight from the
// plan's pinned host copy (visible to the GPU) into the workspace.
__global__ __launch_bounds__(256) void k_header(void **ptab, PtrChunk c, const uint4 *src, uint4 *dst, int64_t n16) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < c.count; i += 256) ptab[c.first + i] = c.p[i];
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += step) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// permuting copy (leaf staging, naive-order re-layout, root permute)

template <typename T>
__global__ void k_copy(const CopyDesc *descs, const void *const *ptab, const int64_t *ints, SliceDigits sd,
                       int32_t beta) {
  const CopyDesc d = descs[blockIdx.y];
  const int64_t *dims = ints + d.ints_index;
  const int64_t *sst = dims + d.rank;
  const int64_t *slc = sst + d.rank;
  int64_t base = d.src_off;
  for (int t = 0; t < sd.n; ++t) base += (int64_t)sd.digit[t] * slc[t];
  const T *src = (const T *)ptab[d.src_buf] + base;
  T *dst = (T *)ptab[d.dst_buf] + d.dst_off;
  const int b = beta && d.is_root;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < d.count; e += step) {
    int64_t r = e, so = 0;
    for (int p = d.rank - 1; p >= 0; --p) {
      const int64_t dm = dims[p];
      so += (r % dm) * sst[p];
      r /= dm;
    }
    store_c(dst + e, src[so], b);
  }
}

// Tiled permuting copy: reads go along the source's smallest strides, writes
// along the destination's innermost dims, with the tile transposed in LDS.
// The per-entry offset tables are built on the host (they hold the index
// arithmetic) and staged into LDS once per workgroup.  Each pass moves NE
// entries (as many whole tiles as fit), NE / 256 independent loads per
// thread between two barriers, so many loads are in flight at once.
constexpr int kTileMax = 1024;

template <typename T, int NE>
__global__ __launch_bounds__(256) void k_copy_tiled(const CopyDesc *desc, const void *const *ptab, const int64_t *ints,
                                                    SliceDigits sd, int32_t beta) {
  constexpr int EPT = NE / 256;
  constexpr int kMaxTilesPerPass = NE / 32;
  constexpr bool kPairsPossible = sizeof(T) == 8;
  __shared__ __align__(16) T buf[NE];
  __shared__ int64_t s_src[kTileMax];
  __shared__ int32_t s_lds[kTileMax];
  __shared__ int64_t s_dst[kTileMax];
  __shared__ int64_t s_bs[kMaxTilesPerPass], s_bd[kMaxTilesPerPass];
  __shared__ int s_pairs;
  const CopyDesc d = *desc;
  const int64_t *t = ints + d.ints_index;
  const int tile = (int)t[0];
  const int nout = (int)t[1];
  const int pow2 = (int)t[2];
  const int64_t *od = t + 3;
  const int64_t *osrc = od + nout;
  const int64_t *odst = osrc + nout;
  const int64_t *slc = odst + nout;
  const int64_t *ld_src = slc + sd.n;
  const int64_t *ld_lds = ld_src + tile;
  const int64_t *st_dst = ld_lds + tile;
  const int tid = threadIdx.x;
  int64_t base = d.src_off;
  for (int q = 0; q < sd.n; ++q) base += (int64_t)sd.digit[q] * slc[q];
  const T *src = (const T *)ptab[d.src_buf] + base;
  T *dst = (T *)ptab[d.dst_buf] + d.dst_off;
  if (tid == 0) {
    // 16-byte pairs: entries 2i, 2i+1 of the tile adjacent in both the
    // source and the destination, every pair and every tile base 16-byte
    // aligned (checked on the tables below)
    int ok = kPairsPossible && (tile % 2) == 0 && aligned16(src) && aligned16(dst);
    for (int q = 0; q < nout && ok; ++q) ok = (osrc[q] % 2) == 0 && (odst[q] % 2) == 0;
    s_pairs = ok;
  }
  __syncthreads();
  for (int e = tid; e < tile; e += blockDim.x) {
    s_src[e] = ld_src[e];
    s_lds[e] = (int32_t)ld_lds[e];
    s_dst[e] = st_dst[e];
    if ((e % 2) == 0 && e + 1 < tile &&
        ((ld_src[e] % 2) != 0 || ld_src[e + 1] != ld_src[e] + 1 || (st_dst[e] % 2) != 0 ||
         st_dst[e + 1] != st_dst[e] + 1))
      s_pairs = 0;
  }
  const int b = beta && d.is_root;
  const int64_t ntiles = d.count / tile;
  const int ut = NE / tile;  // tiles per pass (tile >= 32)
  __syncthreads();
  const bool pairs = s_pairs != 0;
  for (int64_t o0 = (int64_t)blockIdx.x * ut; o0 < ntiles; o0 += (int64_t)gridDim.x * ut) {
    if (tid < ut) {
      int64_t r = o0 + tid, bs = 0, bd = 0;
      if (pow2) {
        for (int q = nout - 1; q >= 0; --q) {
          const int64_t e = od[q];
          bs += (r & (e - 1)) * osrc[q];
          bd += (r & (e - 1)) * odst[q];
          r >>= __builtin_ctzll((unsigned long long)e);
        }
      } else {
        for (int q = nout - 1; q >= 0; --q) {
          const int64_t e = od[q];
          const int64_t dg = r % e;
          r /= e;
          bs += dg * osrc[q];
          bd += dg * odst[q];
        }
      }
      s_bs[tid] = bs;
      s_bd[tid] = bd;
    }
    __syncthreads();
    if (kPairsPossible && pairs) {
#pragma unroll
      for (int j = 0; j < EPT / 2; ++j) {
        const int E = 2 * (tid + 256 * j);
        const int u = E / tile, e = E - u * tile;
        if (u < ut && o0 + u < ntiles) {
          const float4 v = *(const float4 *)(src + s_bs[u] + s_src[e]);
          float2 *bb = (float2 *)buf + u * tile;
          bb[s_lds[e]] = make_float2(v.x, v.y);
          bb[s_lds[e + 1]] = make_float2(v.z, v.w);
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EPT / 2; ++j) {
        const int E = 2 * (tid + 256 * j);
        const int u = E / tile, e = E - u * tile;
        if (u < ut && o0 + u < ntiles) {
          float4 v = *(const float4 *)((float2 *)buf + E);
          float4 *p = (float4 *)(dst + s_bd[u] + s_dst[e]);
          if (b) {
            const float4 o = *p;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *p = v;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int E = tid + 256 * j;
        const int u = E / tile, e = E - u * tile;
        if (u < ut && o0 + u < ntiles) buf[u * tile + s_lds[e]] = src[s_bs[u] + s_src[e]];
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int E = tid + 256 * j;
        const int u = E / tile, e = E - u * tile;
        if (u < ut && o0 + u < ntiles) store_c(dst + s_bd[u] + s_dst[e], buf[E], b);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// grouped tiny steps: one workgroup per step

constexpr int tiny_stage_entries(int bytes) { return bytes == 8 ? 4096 : 2048; }
constexpr int kTinyTable = 256;  // rows (and columns) covered by a member's offset table

// Complex64 member with 32 <= R, S <= 256 whose operands are staged in LDS:
// the four waves take 32 x 32 output blocks in turn, each on the FP32 matrix
// cores with the (re, im) scheme of k_cgemm (lanes 0-31 supply xr and (yr,
// yi), lanes 32-63 xi and (-yi, yr)); row and column offsets of the output
// come from the member's offset table (rows at toff[0..255], columns at
// toff[256..511]).
__device__ __forceinline__ void tiny_member_mfma(const float2 *X, const float2 *Y, float2 *C, int R, int S, int K,
                                                 int b, const int64_t *toff, int part, int parts) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const float *Xf = (const float *)X, *Yf = (const float *)Y;
  const int bc = (S + 31) / 32, nblk = ((R + 31) / 32) * bc;
  for (int blk = wave + 4 * part; blk < nblk; blk += 4 * parts) {
    const int i0 = (blk / bc) * 32, j0 = (blk % bc) * 32;
    const int row = i0 + l32, col = j0 + l32;
    const bool rv = row < R, cv = col < S;
    f32x16 aR, aI;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      aR[r] = 0.f;
      aI[r] = 0.f;
    }
    for (int l = 0; l < K; ++l) {
      const float xa = rv ? Xf[2 * (row * K + l) + h] : 0.f;
      const float yre = cv ? Yf[2 * (col * K + l)] : 0.f;
      const float yim = cv ? Yf[2 * (col * K + l) + 1] : 0.f;
      aR = __builtin_amdgcn_mfma_f32_32x32x2f32(xa, h ? -yim : yre, aR, 0, 0, 0);
      aI = __builtin_amdgcn_mfma_f32_32x32x2f32(xa, h ? yre : yim, aI, 0, 0, 0);
    }
    if (cv) {
      const int64_t co = toff[kTinyTable + col];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gi = i0 + (r / 4) * 8 + h * 4 + (r % 4);
        if (gi < R) store_c(C + toff[gi] + co, make_float2(aR[r], aI[r]), b);
      }
    }
  }
}

// One member of a tiny group, computed by one workgroup.  Both operands of a
// member whose (R + S) K entries fit are first copied into LDS with
// coalesced loads (one round trip), so the passes below read LDS instead of
// waiting on a global load per pass.  A member with R, S <= 256 first tabulates
// the output offsets of its rows and columns (one run walk per row and per
// column instead of two per output).  Ends with a barrier, so `stage` and
// `toff` may be reused by the next member.
template <typename T>
__device__ __forceinline__ void tiny_member(const TinyDesc &d, const void *const *ptab, const RunDev *runs,
                                            int32_t beta, T *stage, int64_t *toff, int part, int parts) {
  constexpr int kStage = tiny_stage_entries(sizeof(T));
  const T *X = (const T *)ptab[d.x_buf] + d.x_off;
  const T *Y = (const T *)ptab[d.y_buf] + d.y_off;
  T *C = (T *)ptab[d.c_buf] + d.c_off;
  const RunDev *rr = runs + d.runs_index;
  const RunDev *cr = rr + d.nrr;
  const int R = d.R, S = d.S, K = d.K;
  const bool table = R <= kTinyTable && S <= kTinyTable;
  const bool staged = (int64_t)(R + S) * K <= kStage;
  if (table)
    for (int t = threadIdx.x; t < 2 * kTinyTable; t += 256)
      toff[t] = t < kTinyTable ? (t < R ? run_offset(t, rr, d.nrr) : 0)
                               : (t - kTinyTable < S ? run_offset(t - kTinyTable, cr, d.ncr) : 0);
  if (staged) {
    const int nx = R * K, ny = S * K;
    for (int e = threadIdx.x; e < nx; e += 256) stage[e] = X[e];
    for (int e = threadIdx.x; e < ny; e += 256) stage[nx + e] = Y[e];
    X = stage;
    Y = stage + nx;
  }
  if (table || staged) __syncthreads();
  if constexpr (sizeof(T) == 8) {
    if (staged && table && R >= 32 && S >= 32) {
      tiny_member_mfma(X, Y, C, R, S, K, beta && d.is_root, toff, part, parts);
      __syncthreads();
      return;
    }
  }
  const int outputs = R * S;
  // lanes per output: a power of two <= 64 that keeps the workgroup busy
  int G = 1;
  while (G < 64 && G * 2 <= K && outputs * G * 2 <= 256) G *= 2;
  const int per_pass = 256 / G;
  const int lane = threadIdx.x % G;
  const int grp = threadIdx.x / G;
  const int b = beta && d.is_root;
  for (int o0 = part * per_pass; o0 < outputs; o0 += per_pass * parts) {
    const int o = o0 + grp;
    T acc = czero<T>();
    if (o < outputs) {
      const int i = o / S, j = o - (o / S) * S;
      const T *xr = X + (int64_t)i * K;
      const T *yr = Y + (int64_t)j * K;
      for (int l = lane; l < K; l += G) cmac(acc, xr[l], yr[l]);
    }
    for (int w = 1; w < G; w *= 2) {
      acc.x += __shfl_xor(acc.x, w, 64);
      acc.y += __shfl_xor(acc.y, w, 64);
    }
    if (o < outputs && lane == 0) {
      const int i = o / S, j = o - (o / S) * S;
      const int64_t off = table ? toff[i] + toff[kTinyTable + j] : run_offset(i, rr, d.nrr) + run_offset(j, cr, d.ncr);
      store_c(C + off, acc, b);
    }
  }
  __syncthreads();
}

// `parts` workgroups per member: workgroup b takes member b / parts and the
// output blocks (or passes) congruent to b % parts.
template <typename T>
__global__ __launch_bounds__(256) void k_tiny(const TinyDesc *descs, const void *const *ptab, const RunDev *runs,
                                              int32_t beta, int parts) {
  __shared__ T stage[tiny_stage_entries(sizeof(T))];
  __shared__ int64_t toff[2 * kTinyTable];
  tiny_member<T>(descs[blockIdx.x / parts], ptab, runs, beta, stage, toff, (int)(blockIdx.x % parts), parts);
}

// ---------------------------------------------------------------------------
// skinny steps: S <= 16 columns, rows streamed from HBM

constexpr int kSkinnyMax = 16;

__device__ __forceinline__ float2 ld_pair_lo(const float4 &v) { return make_float2(v.x, v.y); }
__device__ __forceinline__ float2 ld_pair_hi(const float4 &v) { return make_float2(v.z, v.w); }

// Few rows (R < 4096): one workgroup per (row, K chunk); all 256 threads
// stride over the chunk with 16-byte loads (two entries), accumulate the
// row's S outputs, and reduce through shuffles and LDS.
__global__ __launch_bounds__(256) void k_skinny(StepArgs a, int64_t kchunk) {
  __shared__ float2 red[4][kSkinnyMax];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t k0 = (int64_t)split * kchunk;
  const int64_t k1 = min(a.K, k0 + kchunk);
  const int S = (int)a.S;
  float2 acc[kSkinnyMax];
#pragma unroll
  for (int q = 0; q < kSkinnyMax; ++q) acc[q] = make_float2(0.f, 0.f);
  const float2 *xr = a.X + i * a.K;
  // 16-byte loads need 16-byte aligned row starts; otherwise 8-byte ones
  const bool pairs = aligned16(xr + k0) && aligned16(a.Y + k0) && (a.K % 2 == 0);
  if (pairs) {
    const int64_t np = (k1 - k0) / 2;
    const float4 *x4 = (const float4 *)(xr + k0);
    for (int64_t p = tid; p < np; p += 256) {
      const float4 xv = x4[p];
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S) {
          const float4 yv = ((const float4 *)(a.Y + (int64_t)q * a.K + k0))[p];
          cmac(acc[q], ld_pair_lo(xv), ld_pair_lo(yv));
          cmac(acc[q], ld_pair_hi(xv), ld_pair_hi(yv));
        }
    }
    if ((k1 - k0) % 2 == 1 && tid == 0) {
      const int64_t l = k1 - 1;
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S) cmac(acc[q], xr[l], a.Y[(int64_t)q * a.K + l]);
    }
  } else {
    for (int64_t l = k0 + tid; l < k1; l += 256) {
      const float2 x = xr[l];
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S) cmac(acc[q], x, a.Y[(int64_t)q * a.K + l]);
    }
  }
#pragma unroll
  for (int q = 0; q < kSkinnyMax; ++q) {
    for (int w = 1; w < 64; w *= 2) {
      acc[q].x += __shfl_xor(acc[q].x, w, 64);
      acc[q].y += __shfl_xor(acc[q].y, w, 64);
    }
    if (lane == 0 && q < S) red[wave][q] = acc[q];
  }
  __syncthreads();
  if (tid < S) {
    float2 v = red[0][tid];
    for (int w = 1; w < 4; ++w) {
      v.x += red[w][tid].x;
      v.y += red[w][tid].y;
    }
    if (a.splits > 1) a.scratch[((int64_t)split * a.R + i) * a.S + tid] = v;
    else store_c(a.C + run_offset(i, a.runs, a.nrr) + run_offset(tid, a.runs + a.nrr, a.ncr), v, a.beta);
  }
}

// Many rows: workgroups walk tiles of 256 rows (grid-stride), one row per
// thread.  Each K chunk of a tile goes into LDS (row stride 17 entries,
// conflict-free); when the chunk is the whole K, the tile's rows are one
// contiguous block read with 16-byte loads and the small operand is loaded
// once per workgroup.  The small operand is read from LDS by broadcast and
// each thread keeps its row's <= 16 outputs in registers.  A row-major C
// (one run per side, unit column stride) is written through LDS with
// 16-byte stores; other layouts go through the runs per entry.
constexpr int kRowsKC = 16;

__global__ __launch_bounds__(256) void k_skinny_rows(StepArgs a, int64_t kchunk) {
  __shared__ float2 xs[256][kRowsKC + 1];
  __shared__ float2 ys[kSkinnyMax][kRowsKC];
  __shared__ int64_t coloff[kSkinnyMax];
  const int tid = threadIdx.x;
  const int S = (int)a.S;
  const int64_t K = a.K;
  const int split = blockIdx.y;
  const int64_t k0 = (int64_t)split * kchunk;
  const int64_t k1 = min(K, k0 + kchunk);
  const bool whole = (k0 == 0 && k1 == K && K <= kRowsKC);
  const bool rowmajor = a.splits == 1 && a.nrr == 1 && a.ncr == 1 && a.runs[1].stride == 1 &&
                        a.runs[0].stride == a.S;
  if (tid < S) coloff[tid] = run_offset(tid, a.runs + a.nrr, a.ncr);
  if (whole && tid < kSkinnyMax * kRowsKC) {
    const int sr = tid / kRowsKC, col = tid % kRowsKC;
    ys[sr][col] = (sr < S && col < K) ? a.Y[(int64_t)sr * K + col] : make_float2(0.f, 0.f);
  }
  const int64_t ntiles = (a.R + 255) / 256;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t r0 = tile * 256;
    const int rows = (int)min((int64_t)256, a.R - r0);
    float2 acc[kSkinnyMax];
#pragma unroll
    for (int q = 0; q < kSkinnyMax; ++q) acc[q] = make_float2(0.f, 0.f);
    for (int64_t kc = k0; kc < k1; kc += kRowsKC) {
      const int w = (int)min((int64_t)kRowsKC, k1 - kc);
      __syncthreads();
      if (whole) {
        // rows r0 .. r0+rows-1 of X are one contiguous block of rows*K entries
        const int64_t n = (int64_t)rows * K;
        const float2 *src = a.X + r0 * K;
        if (aligned16(src)) {
          const float4 *src4 = (const float4 *)src;
          for (int64_t p = tid; p < n / 2; p += 256) {
            const float4 v = src4[p];
            const int e = (int)(2 * p);
            xs[e / K][e % K] = ld_pair_lo(v);
            xs[(e + 1) / K][(e + 1) % K] = ld_pair_hi(v);
          }
          if ((n % 2) == 1 && tid == 0) xs[(n - 1) / K][(n - 1) % K] = src[n - 1];
        } else {
          for (int64_t e = tid; e < n; e += 256) xs[e / K][e % K] = src[e];
        }
      } else {
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          const int row = tid / kRowsKC + 16 * p, col = tid % kRowsKC;
          xs[row][col] = (row < rows && col < w) ? a.X[(r0 + row) * K + kc + col] : make_float2(0.f, 0.f);
        }
        if (tid < kSkinnyMax * kRowsKC) {
          const int sr = tid / kRowsKC, col = tid % kRowsKC;
          ys[sr][col] = (sr < S && col < w) ? a.Y[(int64_t)sr * K + kc + col] : make_float2(0.f, 0.f);
        }
      }
      __syncthreads();
      if (tid < rows) {
        for (int l = 0; l < w; ++l) {
          const float2 x = xs[tid][l];
#pragma unroll
          for (int q = 0; q < kSkinnyMax; ++q)
            if (q < S) cmac(acc[q], x, ys[q][l]);
        }
      }
    }
    const int64_t i = r0 + tid;
    if (a.splits > 1) {
      if (tid < rows) {
        float2 *p = a.scratch + ((int64_t)split * a.R + i) * a.S;
#pragma unroll
        for (int q = 0; q < kSkinnyMax; ++q)
          if (q < S) p[q] = acc[q];
      }
    } else if (rowmajor) {
      // the tile's outputs are rows*S contiguous entries: stage them in LDS
      // (xs holds 256 x 17 entries >= 256 x 16) and store 16 bytes per lane
      __syncthreads();
      float2 *stage = &xs[0][0];
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S && tid < rows) stage[tid * S + q] = acc[q];
      __syncthreads();
      const int64_t n = (int64_t)rows * S;
      float2 *dst = a.C + a.runs[0].stride * r0;
      if (aligned16(dst)) {
        for (int64_t p = tid; p < n / 2; p += 256) {
          float2 lo = stage[2 * p], hi = stage[2 * p + 1];
          if (a.beta) {
            const float4 o = ((const float4 *)dst)[p];
            lo.x += o.x; lo.y += o.y; hi.x += o.z; hi.y += o.w;
          }
          ((float4 *)dst)[p] = make_float4(lo.x, lo.y, hi.x, hi.y);
        }
        if ((n % 2) == 1 && tid == 0) store_c(dst + n - 1, stage[n - 1], a.beta);
      } else {
        for (int64_t e = tid; e < n; e += 256) store_c(dst + e, stage[e], a.beta);
      }
    } else if (tid < rows) {
      const int64_t ro = run_offset(i, a.runs, a.nrr);
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S) store_c(a.C + ro + coloff[q], acc[q], a.beta);
    }
  }
}

// Outer products (K = 1, at most kSkinnyMax outputs per row) of a long
// operand: C at rowoff(i) + coloff(j) = X[i] Y[j], pure streaming.  When C's
// innermost row run has stride 1 and an even size, rows 2p and 2p + 1 sit
// side by side in C and every other stride is even, so each lane reads a
// row pair with one 16-byte load and writes one 16-byte pair per output
// column; otherwise it takes single rows.  Grid-stride over chunks of 256 U
// row pairs (U loads in flight per lane), no LDS staging of X.
constexpr int kOuterU = 4;
__global__ __launch_bounds__(256) void k_outer(StepArgs a) {
  __shared__ float2 ys[kSkinnyMax];
  __shared__ int64_t coloff[kSkinnyMax];
  const int tid = threadIdx.x, S = (int)a.S;
  if (tid < S) {
    ys[tid] = a.Y[tid];
    coloff[tid] = run_offset(tid, a.runs + a.nrr, a.ncr);
  }
  __syncthreads();
  const RunDev inner = a.runs[a.nrr - 1];
  const bool pairs = a.nrr >= 1 && inner.stride == 1 && (inner.size % 2) == 0 && (a.R % 2) == 0 &&
                     aligned16(a.X) && aligned16(a.C);
  if (pairs) {
    const int64_t np = a.R / 2;
    const float4 *X4 = (const float4 *)a.X;
    for (int64_t base = (int64_t)blockIdx.x * 256 * kOuterU; base < np;
         base += (int64_t)gridDim.x * 256 * kOuterU) {
      float4 v[kOuterU];
#pragma unroll
      for (int u = 0; u < kOuterU; ++u) {
        const int64_t p = base + u * 256 + tid;
        if (p < np) v[u] = X4[p];
      }
#pragma unroll
      for (int u = 0; u < kOuterU; ++u) {
        const int64_t p = base + u * 256 + tid;
        if (p >= np) continue;
        const int64_t ro = run_offset(2 * p, a.runs, a.nrr);
        for (int j = 0; j < S; ++j) {
          const float2 y = ys[j];
          float4 o = make_float4(v[u].x * y.x - v[u].y * y.y, v[u].x * y.y + v[u].y * y.x,
                                 v[u].z * y.x - v[u].w * y.y, v[u].z * y.y + v[u].w * y.x);
          float4 *dst = (float4 *)(a.C + ro + coloff[j]);
          if (a.beta) {
            const float4 c = *dst;
            o.x += c.x; o.y += c.y; o.z += c.z; o.w += c.w;
          }
          *dst = o;
        }
      }
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < a.R; i += (int64_t)gridDim.x * 256) {
      const float2 x = a.X[i];
      const int64_t ro = run_offset(i, a.runs, a.nrr);
      for (int j = 0; j < S; ++j) {
        const float2 y = ys[j];
        store_c(a.C + ro + coloff[j], make_float2(x.x * y.x - x.y * y.y, x.x * y.y + x.y * y.x), a.beta);
      }
    }
  }
}

// Many rows, whole K <= 16, no split: no LDS staging of X at all.  Each
// thread streams ROWS rows (row r of the step is row
// (blockIdx.x * ROWS + u) * 256 + tid, so every u is a coalesced group of
// 256 rows) with 16-byte loads where aligned, keeps every output in
// registers, and reads the small operand from LDS by broadcast.  No barrier
// inside the loop, so many waves keep loads in flight.
template <int ROWS>
__global__ __launch_bounds__(256) void k_skinny_small(StepArgs a) {
  static_assert(ROWS >= 1 && ROWS <= 2, "rows per thread");
  __shared__ float2 ys[kSkinnyMax][kRowsKC];
  __shared__ int64_t coloff[kSkinnyMax];
  const int tid = threadIdx.x;
  const int K = (int)a.K, S = (int)a.S;
  if (tid < kSkinnyMax * kRowsKC) {
    const int sr = tid / kRowsKC, col = tid % kRowsKC;
    ys[sr][col] = (sr < S && col < K) ? a.Y[(int64_t)sr * K + col] : make_float2(0.f, 0.f);
  }
  if (tid < S) coloff[tid] = run_offset(tid, a.runs + a.nrr, a.ncr);
  __syncthreads();
  const bool rowmajor = a.nrr == 1 && a.ncr == 1 && a.runs[1].stride == 1 && a.runs[0].stride == a.S;
  float2 x[ROWS][kRowsKC];
  int64_t row[ROWS];
#pragma unroll
  for (int u = 0; u < ROWS; ++u) {
    row[u] = ((int64_t)blockIdx.x * ROWS + u) * 256 + tid;
    const float2 *src = a.X + row[u] * K;
    if (row[u] < a.R) {
      if ((K % 2) == 0 && aligned16(src)) {
#pragma unroll
        for (int l = 0; l < kRowsKC; l += 2)
          if (l < K) {
            const float4 v = *(const float4 *)(src + l);
            x[u][l] = ld_pair_lo(v);
            x[u][l + 1] = ld_pair_hi(v);
          }
      } else {
#pragma unroll
        for (int l = 0; l < kRowsKC; ++l)
          if (l < K) x[u][l] = src[l];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < ROWS; ++u) {
    if (row[u] >= a.R) continue;
    float2 acc[kSkinnyMax];
#pragma unroll
    for (int q = 0; q < kSkinnyMax; ++q) {
      acc[q] = make_float2(0.f, 0.f);
      if (q < S) {
#pragma unroll
        for (int l = 0; l < kRowsKC; ++l)
          if (l < K) cmac(acc[q], x[u][l], ys[q][l]);
      }
    }
    if (rowmajor) {
      float2 *dst = a.C + row[u] * a.S;
      if ((S % 2) == 0 && aligned16(dst)) {
#pragma unroll
        for (int q = 0; q < kSkinnyMax; q += 2)
          if (q < S) {
            float2 lo = acc[q], hi = acc[q + 1];
            if (a.beta) {
              const float4 o = *(const float4 *)(dst + q);
              lo.x += o.x; lo.y += o.y; hi.x += o.z; hi.y += o.w;
            }
            *(float4 *)(dst + q) = make_float4(lo.x, lo.y, hi.x, hi.y);
          }
      } else {
#pragma unroll
        for (int q = 0; q < kSkinnyMax; ++q)
          if (q < S) store_c(dst + q, acc[q], a.beta);
      }
    } else {
      const int64_t ro = run_offset(row[u], a.runs, a.nrr);
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S) store_c(a.C + ro + coloff[q], acc[q], a.beta);
    }
  }
}

// Many rows, whole K a power of two in [2, 256], S <= 16: the rows of X are
// one contiguous stream and no barrier or LDS staging of X is needed.  G
// lanes share a row; lane p of a row reads the 16-byte chunks p, p + G, ...
// (V of them, so a wave's loads cover whole rows) and forms partial sums of
// all SP outputs (S padded to a power of two; padded Y rows are zero) over
// its 2V entries of K.  The G partials are combined with DPP lane exchanges
// inside each 16-lane row: first all-reduce steps while the lanes outnumber
// the outputs, then reduce-scatter steps, each of which halves the outputs a
// lane keeps, so lane p ends with SP/G consecutive outputs and a row-major C
// is written by contiguous lanes.  The small operand sits in registers when
// it fits, else in LDS (row stride SP + 1, conflict-free).
constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v / 2); }
constexpr int dpp_ctrl_for_bit(int b) {
  // partner lane of each exchange flips the lane-index bit b (and only
  // lower bits): row_mirror (i <-> 15 - i), row_half_mirror (i <-> 7 - i
  // within 8), quad_perm [2,3,0,1], quad_perm [1,0,3,2]
  return b == 8 ? 0x140 : b == 4 ? 0x141 : b == 2 ? 0x4E : 0xB1;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// all-reduce step: both lanes of a pair end with the pair's sum of all N
template <int CTRL, int N>
__device__ __forceinline__ void xchg_all(float *re, float *im) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    re[j] += dpp_f<CTRL>(re[j]);
    im[j] += dpp_f<CTRL>(im[j]);
  }
}

// reduce-scatter step: the lane with the pair bit set keeps the upper half
// of its N values, its partner the lower half; each sends the half it drops
template <int CTRL, int N>
__device__ __forceinline__ void xchg_scatter(float *re, float *im, bool upper) {
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const float sr = upper ? re[j] : re[j + N / 2], si = upper ? im[j] : im[j + N / 2];
    const float kr = upper ? re[j + N / 2] : re[j], ki = upper ? im[j + N / 2] : im[j];
    re[j] = kr + dpp_f<CTRL>(sr);
    im[j] = ki + dpp_f<CTRL>(si);
  }
}

template <int BIT, int AR, int N>
__device__ __forceinline__ void xchg_group(float *re, float *im, int lpos) {
  if constexpr (BIT >= 1) {
    if constexpr (AR > 0) {
      xchg_all<dpp_ctrl_for_bit(BIT), N>(re, im);
      xchg_group<BIT / 2, AR - 1, N>(re, im, lpos);
    } else {
      xchg_scatter<dpp_ctrl_for_bit(BIT), N>(re, im, (lpos & BIT) != 0);
      xchg_group<BIT / 2, 0, N / 2>(re, im, lpos);
    }
  }
}

constexpr int flat_lanes(int K, int SP) {
  int g = SP > K / 16 ? SP : K / 16;
  if (g > K / 2) g = K / 2;
  if (g > 16) g = 16;
  return g < 1 ? 1 : g;
}

template <int G, int V, int SP, bool YREG, int U>
__global__ __launch_bounds__(256) void k_skinny_flat(StepArgs a) {
  constexpr int KH = G * V;                 // 16-byte chunks (entry pairs) per row
  constexpr int K = 2 * KH;
  constexpr int RPB = 256 / G;              // rows per workgroup pass
  constexpr int LG = ilog2c(G), LS = ilog2c(SP);
  constexpr int RS = LG < LS ? LG : LS;     // reduce-scatter steps
  constexpr int NOUT = SP >> RS;            // outputs a lane keeps
  constexpr int GS = G < SP ? G : SP;       // lanes that hold distinct outputs
  __shared__ float4 ysl[YREG ? 1 : KH * (SP + 1)];
  __shared__ int64_t coloff[kSkinnyMax];
  const int tid = threadIdx.x, lpos = tid % G;
  const int S = (int)a.S;
  const bool rowmajor = a.nrr == 1 && a.ncr == 1 && a.runs[1].stride == 1 && a.runs[0].stride == a.S;
  if (tid < S) coloff[tid] = run_offset(tid, a.runs + a.nrr, a.ncr);
  float4 yr[YREG ? V : 1][YREG ? SP : 1];
  if constexpr (YREG) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c = lpos + G * v;
#pragma unroll
      for (int q = 0; q < SP; ++q) {
        if (q < S) {
          const float2 y0 = a.Y[(int64_t)q * K + 2 * c], y1 = a.Y[(int64_t)q * K + 2 * c + 1];
          yr[v][q] = make_float4(y0.x, y0.y, y1.x, y1.y);
        } else {
          yr[v][q] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  } else {
    for (int e = tid; e < KH * SP; e += 256) {
      const int c = e / SP, q = e % SP;
      float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
      if (q < S) {
        const float2 y0 = a.Y[(int64_t)q * K + 2 * c], y1 = a.Y[(int64_t)q * K + 2 * c + 1];
        y = make_float4(y0.x, y0.y, y1.x, y1.y);
      }
      ysl[c * (SP + 1) + q] = y;
    }
  }
  __syncthreads();
  const float4 *X4 = (const float4 *)a.X;
  const int64_t R = a.R;
  const int64_t stride = (int64_t)gridDim.x * RPB;
  const bool pairs = (NOUT % 2) == 0 && S == SP && aligned16(a.C);
  for (int64_t r0 = (int64_t)blockIdx.x * RPB + tid / G; r0 < R; r0 += stride * U) {
    float4 xv[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rr = r0 + u * stride;
#pragma unroll
      for (int v = 0; v < V; ++v)
        xv[u][v] = rr < R ? X4[rr * KH + lpos + G * v] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // re-read the LDS copy of the small operand every pass (an opaque
    // index stops the compiler from hoisting all V * SP reads into registers)
    int cb = lpos;
    if constexpr (!YREG) asm volatile("" : "+v"(cb));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rr = r0 + u * stride;
      float re[SP], im[SP];
#pragma unroll
      for (int q = 0; q < SP; ++q) re[q] = im[q] = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float4 x = xv[u][v];
#pragma unroll
        for (int q = 0; q < SP; ++q) {
          const float4 y = YREG ? yr[v < V ? v : 0][q] : ysl[(cb + G * v) * (SP + 1) + q];
          re[q] = fmaf(x.x, y.x, re[q]);
          re[q] = fmaf(-x.y, y.y, re[q]);
          re[q] = fmaf(x.z, y.z, re[q]);
          re[q] = fmaf(-x.w, y.w, re[q]);
          im[q] = fmaf(x.x, y.y, im[q]);
          im[q] = fmaf(x.y, y.x, im[q]);
          im[q] = fmaf(x.z, y.w, im[q]);
          im[q] = fmaf(x.w, y.z, im[q]);
        }
      }
      xchg_group<G / 2, LG - RS, SP>(re, im, lpos);
      if (rr < R && (G <= SP || lpos < SP)) {
        const int base = (lpos % GS) * NOUT;
        if (rowmajor) {
          float2 *dst = a.C + rr * S + base;
          if (pairs) {
#pragma unroll
            for (int j = 0; j < NOUT; j += 2) {
              float4 o = make_float4(re[j], im[j], re[j + 1], im[j + 1]);
              if (a.beta) {
                const float4 c = *(const float4 *)(dst + j);
                o.x += c.x; o.y += c.y; o.z += c.z; o.w += c.w;
              }
              *(float4 *)(dst + j) = o;
            }
          } else {
#pragma unroll
            for (int j = 0; j < NOUT; ++j)
              if (base + j < S) store_c(dst + j, make_float2(re[j], im[j]), a.beta);
          }
        } else {
          const int64_t ro = run_offset(rr, a.runs, a.nrr);
#pragma unroll
          for (int j = 0; j < NOUT; ++j)
            if (base + j < S) store_c(a.C + ro + coloff[base + j], make_float2(re[j], im[j]), a.beta);
        }
      }
    }
  }
}

// Skinny steps with many rows, S <= 32 outputs per row (a power of two),
// K a power of two (up to 64 for S <= 16, 8 for S = 32), on the FP32
// matrix cores, written in address order.  Also takes GEMM-class steps whose
// short side is at most 32, with the operands (and C's row and column runs)
// exchanged when the long side is the column side.
//
// Each wave owns passes of NB blocks of 32 rows: it loads the pass's X rows
// (one contiguous stretch of 32 NB K entries) with coalesced 16-byte loads
// into a wave-private LDS area, runs the MFMAs over it and writes the
// results back into the same area (LDS operations of one wave complete in
// order, so no barrier is needed).  With SW = 16 the 32 MFMA columns carry
// the real parts of the S outputs (columns 0-15) and their imaginary parts
// (16-31): with the (re, im) K-slot scheme of k_cgemm, column j < 16 takes
// (yr, -yi) of output j and column 16 + j takes (yi, yr), so one MFMA per
// complex entry of K yields both parts.  With SW = 32 the real and the
// imaginary parts take one MFMA each, as in k_cgemm.  With SW = 8 (S <= 8)
// the 16 x 16 x 4 MFMA takes an entry pair per instruction: lane group
// g = lane / 16 supplies K slot g of (re, im, re', im'), read from LDS as
// one float, and its 16 columns carry the real (0-7) and imaginary (8-15)
// parts, with second operands (yr, -yi, yr', -yi') and (yi, yr, yi', yr').
// The next pass's loads are issued before this pass's MFMAs and stores.
//
// Stores: when every run of C has a power-of-two size, the offset of row
// r0 + t (r0 a multiple of the pass) is rowoff(r0) + rowoff(t), so the
// pass's outputs sit at rowoff(r0) + rowoff(t) + coloff(j), and the offset
// is a sum of one stride per set bit of (t, j).  Ordering those bits by
// stride gives a fixed permutation of the pass's entries into ascending
// addresses; the wave stores the pass in that order, so lanes write
// consecutive addresses wherever C is contiguous (16-byte pairs when the
// smallest stride is one entry), whatever the interleaving of C's modes.
constexpr int kSmRows = 32;

struct SkinnyRuns {
  const RunDev *rows;  // C's runs over the row (long) side, outermost first
  const RunDev *cols;  // over the column (short) side
  int32_t nr, nc;
};

// NB 32-row sub-blocks per wave pass (NB * S <= 32 for SW = 16): small K and
// S move few bytes per block, so a wave takes several blocks per pass.
template <int K, int NB, int SW>
__global__ __launch_bounds__(256) void k_skinny_mfma(StepArgs a, SkinnyRuns rn) {
  constexpr int KH = K / 2;                  // 16-byte entry pairs per X row
  constexpr int RSX = KH + 1;                // LDS row stride (16-byte units), one pad
  constexpr int ROWS = kSmRows * NB;         // rows per wave pass
  constexpr int XW = ROWS * RSX;             // X rows of one pass
  // ROWS x S complex results with an odd row stride S + 1, so that a walk
  // down a column (the store order when a row mode has the smallest
  // stride) spreads over the LDS banks; NB S <= 32
  constexpr int SMAX = SW == 32 ? 32 : (32 / NB < SW ? 32 / NB : SW);
  constexpr int CW = (ROWS * (SMAX + 1) + 1) / 2;
  constexpr int WB = XW > CW ? XW : CW;
  constexpr int LPT = (ROWS * KH + 63) / 64;  // 16-byte loads per lane per pass
  constexpr int LB = 5 + (NB >= 8 ? 3 : NB >= 4 ? 2 : NB >= 2 ? 1 : 0);  // row bits of a pass
  constexpr int JB = SW == 32 ? 5 : 4;       // column bits of a permutation entry
  static_assert(SW != 32 || K <= 8, "32-wide steps with K > 8 run on k_thin_mfma");
  constexpr int RT = ROWS / 16;              // 16-row tiles of a pass (SW = 8)
  __shared__ float4 buf[4][WB];
  __shared__ int64_t rowoff[ROWS], coloff[32];
  __shared__ uint16_t perm[kSmRows * 32];
  __shared__ int32_t bit_of[13];
  __shared__ int32_t nbits_s, pairs_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int S = (int)a.S;
  const int sb = 31 - __clz(S);  // S is a power of two
  const int SP = S + 1;          // LDS row stride of the staged results
  for (int t = tid; t < ROWS + 32; t += 256) {
    if (t < ROWS) rowoff[t] = run_offset(t, rn.rows, rn.nr);
    else coloff[t - ROWS] = t - ROWS < S ? run_offset(t - ROWS, rn.cols, rn.nc) : 0;
  }
  __syncthreads();
  if (tid == 0) {
    // permutation bits: bits 0 .. sb-1 of an entry index are its column, bits JB .. JB+LB-1 its row
    int64_t st[13];
    int pb[13], nb = 0;
    for (int b = 0; b < sb; ++b) {
      st[nb] = coloff[1 << b];
      pb[nb++] = b;
    }
    for (int b = 0; b < LB; ++b) {
      st[nb] = rowoff[1 << b];
      pb[nb++] = JB + b;
    }
    for (int i = 1; i < nb; ++i)
      for (int q = i; q > 0 && st[q] < st[q - 1]; --q) {
        const int64_t ts = st[q];
        st[q] = st[q - 1];
        st[q - 1] = ts;
        const int tp = pb[q];
        pb[q] = pb[q - 1];
        pb[q - 1] = tp;
      }
    for (int i = 0; i < nb; ++i) bit_of[i] = pb[i];
    nbits_s = nb;
    pairs_s = nb > 0 && st[0] == 1;
  }
  __syncthreads();
  const int nent = ROWS << sb;
  for (int e = tid; e < nent; e += 256) {
    int p = 0;
    for (int i = 0; i < nbits_s; ++i)
      if ((e >> i) & 1) p |= 1 << bit_of[i];
    perm[e] = (uint16_t)p;
  }
  // second operand, per lane and K entry (SW = 8: per lane and entry pair)
  float bv[SW == 8 ? 1 : K], bw[SW == 32 ? K : 1], bv8[SW == 8 ? KH : 1];
  if constexpr (SW == 8) {
    // 16 x 16 x 4 MFMA: lane group g = lane / 16 supplies K slot g of an entry
    // pair, (re, im, re, im); column c = lane % 16 carries the real part of
    // output c (c < 8) or the imaginary part of output c - 8
    const int g = lane >> 4, c = lane & 15, j = c & 7;
#pragma unroll
    for (int q = 0; q < KH; ++q) {
      float2 y0 = make_float2(0.f, 0.f), y1 = y0;
      if (j < S) {
        y0 = a.Y[(int64_t)j * K + 2 * q];
        y1 = a.Y[(int64_t)j * K + 2 * q + 1];
      }
      // slot g: (yr, -yi, yr', -yi') for a real-part column, (yi, yr, yi', yr') for an imaginary one
      const float2 y = g < 2 ? y0 : y1;
      const bool odd = (g & 1) != 0;
      bv8[q] = c < 8 ? (odd ? -y.y : y.x) : (odd ? y.x : y.y);
    }
  } else if constexpr (SW == 16) {
    // MFMA column l32 = (real | imaginary part of output l32 % 16)
    const int j = l32 & 15;
    const bool imc = l32 >= 16;
#pragma unroll
    for (int l = 0; l < K; ++l) {
      const float2 y = j < S ? a.Y[(int64_t)j * K + l] : make_float2(0.f, 0.f);
      bv[l] = imc ? (h ? y.x : y.y) : (h ? -y.y : y.x);
    }
  } else {
    // MFMA column l32 = output l32: (yr, -yi) for the real part, (yi, yr) for the imaginary part
#pragma unroll
    for (int l = 0; l < K; ++l) {
      const float2 y = l32 < S ? a.Y[(int64_t)l32 * K + l] : make_float2(0.f, 0.f);
      bv[l] = h ? -y.y : y.x;
      bw[l] = h ? y.x : y.y;
    }
  }
  __syncthreads();
  const bool pairs = pairs_s && aligned16(a.C);
  const int64_t R = a.R, npass = (R + ROWS - 1) / ROWS;
  const int64_t wstride = (int64_t)gridDim.x * 4;
  const int64_t lim = R * KH;
  const float4 *X4 = (const float4 *)a.X;
  float4 *xb = buf[wave];
  float4 ld[LPT];
  auto load = [&](int64_t b) {
    const int64_t base = b * ROWS * KH;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int g = lane + 64 * i;
      ld[i] = (g < ROWS * KH && base + g < lim) ? X4[base + g] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  int64_t blk = (int64_t)blockIdx.x * 4 + wave;
  if (blk < npass) load(blk);
  for (; blk < npass; blk += wstride) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int g = lane + 64 * i;
      if (g < ROWS * KH) xb[(g / KH) * RSX + g % KH] = ld[i];
    }
    if (blk + wstride < npass) load(blk + wstride);
    f32x16 acc[SW == 8 ? 1 : NB], acw[SW == 32 ? NB : 1];
    f32x4 acc8[SW == 8 ? RT : 1];
    if constexpr (SW == 8) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc8[t][r] = 0.f;
      // A operand: row t * 16 + lane % 16, K slot lane / 16 of the pair, one
      // 4-byte LDS read
      const float *xf = (const float *)xb;
#pragma unroll
      for (int q = 0; q < KH; ++q)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const float av = xf[((t * 16 + (lane & 15)) * RSX + q) * 4 + (lane >> 4)];
          acc8[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv8[q], acc8[t], 0, 0, 0);
        }
    } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[nb][r] = 0.f;
        if constexpr (SW == 32) acw[nb][r] = 0.f;
      }
#pragma unroll
    for (int q = 0; q < KH; ++q) {
      const float b0 = bv[2 * q], b1 = bv[2 * q + 1];
      float w0 = 0.f, w1 = 0.f;
      if constexpr (SW == 32) {
        w0 = bw[2 * q];
        w1 = bw[2 * q + 1];
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float4 f = xb[(nb * kSmRows + l32) * RSX + q];
        const float x0 = h ? f.y : f.x, x1 = h ? f.w : f.z;
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, b0, acc[nb], 0, 0, 0);
        if constexpr (SW == 32) acw[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, w0, acw[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, b1, acc[nb], 0, 0, 0);
        if constexpr (SW == 32) acw[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, w1, acw[nb], 0, 0, 0);
      }
    }
    }
    // results as complex [ROWS][S] in the same LDS area
    float *cf = (float *)xb;
    const float2 *cv = (const float2 *)xb;
    if constexpr (SW == 8) {
      // 16 x 16 result tile t: lane holds rows t * 16 + 4 (lane / 16) + r of column lane % 16
      const int c = lane & 15, j = c & 7, part = c >> 3;
      if (j < S) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) cf[((t * 16 + 4 * (lane >> 4) + r) * SP + j) * 2 + part] = acc8[t][r];
      }
    } else if constexpr (SW == 16) {
      const int j = l32 & 15, part = l32 >> 4;
      if (j < S) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cf[((nb * kSmRows + (r / 4) * 8 + h * 4 + (r % 4)) * SP + j) * 2 + part] = acc[nb][r];
      }
    } else {
      if (l32 < S) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            *(float2 *)&cf[((nb * kSmRows + (r / 4) * 8 + h * 4 + (r % 4)) * SP + l32) * 2] =
                make_float2(acc[nb][r], acw[nb][r]);
      }
    }
    const int64_t r0 = blk * ROWS;
    const int64_t base = run_offset(r0, rn.rows, rn.nr);
    const int rows = (int)(R - r0 < ROWS ? R - r0 : ROWS);
    constexpr int JM = (1 << JB) - 1;
    if (pairs) {
      for (int e = 2 * lane; e < nent; e += 128) {
        const int p0 = perm[e], p1 = perm[e + 1];
        const int t0 = p0 >> JB, j0 = p0 & JM, t1 = p1 >> JB, j1 = p1 & JM;
        const int64_t o0 = base + rowoff[t0] + coloff[j0];
        const float2 v0 = cv[t0 * SP + j0], v1 = cv[t1 * SP + j1];
        if (t0 < rows && t1 < rows && (o0 & 1) == 0) {
          float4 v = make_float4(v0.x, v0.y, v1.x, v1.y);
          float4 *dst = (float4 *)(a.C + o0);
          if (a.beta) {
            const float4 c = *dst;
            v.x += c.x; v.y += c.y; v.z += c.z; v.w += c.w;
          }
          *dst = v;
        } else {
          if (t0 < rows) store_c(a.C + o0, v0, a.beta);
          if (t1 < rows) store_c(a.C + base + rowoff[t1] + coloff[j1], v1, a.beta);
        }
      }
    } else {
      for (int e = lane; e < nent; e += 64) {
        const int p = perm[e];
        const int t = p >> JB, j = p & JM;
        if (t < rows) store_c(a.C + base + rowoff[t] + coloff[j], cv[t * SP + j], a.beta);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Two chained skinny-class steps in one pass (k_fused2; see Fused2Args).
//
// A long tensor T absorbs a small W1 (K1 = S1 = 4, 8, 16 or 32 entries) and
// the product T1 is reduced at once against another small W2 (K2 = S2).  With
// every mode of extent 2 and the lifetime order of the operands, the modes
// the second step reduces sit right above the first step's reduced modes in
// T, so a block of consecutive rows of T yields whole rows of T1 for the
// second step (the planner checks this per pair).  Each wave takes passes of
// 1024 entries of T: it multiplies the block by W1 on the matrix cores (one
// 32x32x2 MFMA per complex entry of K for 16 outputs, real and imaginary
// parts in the two column halves; two MFMAs for 32 outputs, as in
// k_skinny_mfma), writes the products into its LDS block at their places in
// the second step's rows, multiplies those by W2 and stores T2 in address
// order (the pass's fixed permutation, as in k_skinny_mfma).  T1 never
// reaches HBM: the pair reads T and writes T2 once, half the bytes of the two
// steps run one after the other.  The second operands sit in LDS, one float
// per lane and K entry in the MFMA's column order.  Every LDS write of a pass
// consumes MFMA results that need all of the block's earlier reads, and LDS
// operations of one wave complete in order, so the block is reused in place
// with no barrier; the next pass's loads are issued before this pass's
// MFMAs.  Pairs with K1, K2 <= 8 (the gate steps of state-vector trees) run
// both phases on the vector ALU instead, one lane per row of a block: the
// 32-wide MFMA tile would hold all 1024 / K rows' accumulators at once, and
// at 4 or 8 multiply-adds per entry the ALU keeps up with HBM.

// second-operand table of one phase (K = S): lane l of K entry q at [q][l];
// with K = 32 the imaginary-part columns follow at [K + q][l]
template <int K>
__device__ __forceinline__ void fused_btable(const float2 *W, float *bt, int tid) {
  for (int e = tid; e < K * 64; e += 256) {
    const int l = e >> 6, ln = e & 63, hh = ln >> 5, c = ln & 31;
    if constexpr (K == 32) {
      const float2 y = W[c * K + l];
      bt[e] = hh ? -y.y : y.x;
      bt[K * 64 + e] = hh ? y.x : y.y;
    } else {
      const float2 y = W[(c & 15) * K + l];
      bt[e] = c >= 16 ? (hh ? y.x : y.y) : (hh ? -y.y : y.x);
    }
  }
}

// one phase: NB blocks of 32 rows [row][K / 2 + 1 entry pairs] times the
// table; K = 16: acc holds (re | im) of 16 outputs, K = 32: acc re, acw im
template <int K, int NB>
__device__ __forceinline__ void fused_phase(const float4 *xb, const float *bt, int lane, f32x16 (&acc)[NB],
                                            f32x16 (&acw)[NB]) {
  constexpr int RS = K / 2 + 1;
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[nb][r] = 0.f;
      acw[nb][r] = 0.f;
    }
#pragma unroll
  for (int q = 0; q < K / 2; ++q) {
    const float b0 = bt[(2 * q) * 64 + lane], b1 = bt[(2 * q + 1) * 64 + lane];
    float w0 = 0.f, w1 = 0.f;
    if constexpr (K == 32) {
      w0 = bt[(K + 2 * q) * 64 + lane];
      w1 = bt[(K + 2 * q + 1) * 64 + lane];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float4 f = xb[(nb * 32 + l32) * RS + q];
      const float x0 = h ? f.y : f.x, x1 = h ? f.w : f.z;
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, b0, acc[nb], 0, 0, 0);
      if constexpr (K == 32) acw[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, w0, acw[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, b1, acc[nb], 0, 0, 0);
      if constexpr (K == 32) acw[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, w1, acw[nb], 0, 0, 0);
    }
  }
}

// The part of a vector-ALU phase's product place set by the bits of i (a
// lane takes block rows lane + 64 i; the lane's own bits 0 .. 5 are added
// separately): row bits 6 .. 8 of the block.
__device__ __forceinline__ int fused_rowhi(const int32_t *prow, int i) {
  return ((i & 1) ? prow[6] : 0) + ((i & 2) ? prow[7] : 0) + ((i & 4) ? prow[8] : 0);
}

// A middle step of a fused chain on the vector ALU: lane l takes block rows
// l + 64 i of the step's block xb ([1024 / K rows][K / 2 + 1 entry pairs]),
// multiplies them by the step's table w ([K][K] complex, output rows) and
// writes each product to its place in the next step's block x2: the block
// row's bits through prow, the column's through pcol.  All of the lane's
// reads of xb come before its first write.  wo is an opaque zero that keeps
// the table reads inside the pass loop.
template <int K>
__device__ __forceinline__ void fused_mid_step(const float4 *xb, float2 *x2, const float2 *w, int lane, int wo,
                                               const int32_t *prow, const int32_t *pcol) {
  constexpr int RPL = kFuseEntries / K / 64, RS = K / 2 + 1, LK = K == 8 ? 3 : K == 4 ? 2 : 1;
  float2 z[RPL][K];
#pragma unroll
  for (int i = 0; i < RPL; ++i)
#pragma unroll
    for (int q = 0; q < K / 2; ++q) {
      const float4 f = xb[(lane + 64 * i) * RS + q];
      z[i][2 * q] = make_float2(f.x, f.y);
      z[i][2 * q + 1] = make_float2(f.z, f.w);
    }
  int lp = wo;
#pragma unroll
  for (int b = 0; b < 6; ++b)
    if ((lane >> b) & 1) lp += prow[b];
#pragma unroll
  for (int s = 0; s < K; ++s) {
    float2 wr[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wr[k] = w[s * K + k];
    int pc = 0;
#pragma unroll
    for (int c = 0; c < LK; ++c)
      if ((s >> c) & 1) pc += pcol[c];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      float2 y = make_float2(0.f, 0.f);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        y.x += z[i][k].x * wr[k].x - z[i][k].y * wr[k].y;
        y.y += z[i][k].x * wr[k].y + z[i][k].y * wr[k].x;
      }
      x2[lp + fused_rowhi(prow, i) + pc] = y;
    }
  }
}

// K3 != 0: a chain of three or more steps; its middle steps all have K2,
// or with K2 = 0 take their K (2, 4 or 8) from a.kmid at run time.
template <int K1, int K2, int K3>
__global__ __launch_bounds__(256) void k_fused2(Fused2Args a) {
  constexpr int E = kFuseEntries;
  constexpr int KL = K3 ? K3 : K2;  // the last phase's K (K3 = 0: a pair)
  static_assert(K2 != 0 || K3 != 0, "K2 = 0: a chain whose middle steps take their K at run time");
  constexpr int K2E = K2 ? K2 : 2;  // a chain's middle blocks are at most those of K = 2
  constexpr int ROWS1 = E / K1, ROWS2 = E / K2E, ROWS3 = K3 ? E / K3 : 1, ROWSL = E / KL;
  constexpr int NB1 = ROWS1 / 32, NB2 = ROWS2 / 32;
  constexpr int RS1 = K1 / 2 + 1, RS2 = K2E / 2 + 1, RS3 = K3 / 2 + 1;  // 16-byte units per LDS row, one pad
  constexpr int SP = KL + 1;                         // staged products: complex entries per row
  constexpr int W1F = ROWS1 * RS1, W2F = ROWS2 * RS2, W3F = (ROWSL * SP + 1) / 2, W4F = K3 ? ROWS3 * RS3 : 0;
  constexpr int WB12 = W1F > W2F ? W1F : W2F, WB34 = W3F > W4F ? W3F : W4F;
  constexpr int WB = WB12 > WB34 ? WB12 : WB34;
  constexpr int LPT = E / 2 / 64;  // 16-byte loads per lane per pass
  constexpr int JB2 = KL == 32 ? 5 : KL == 16 ? 4 : KL == 8 ? 3 : KL == 4 ? 2 : 1, LB2 = 10 - JB2;  // the stored product's bits
  constexpr int LKH = K1 == 32 ? 4 : K1 == 16 ? 3 : K1 == 8 ? 2 : K1 == 4 ? 1 : 0;  // log2(K1 / 2)
  constexpr int LB1 = 9 - LKH;            // log2(ROWS1): the pass's local row bits
  constexpr int NPT = 4 * E / 2 / 256;    // store pairs per thread in a workgroup round
  // a phase with K <= 8 runs on the vector ALU, a lane per row (the 32-wide
  // MFMA tile would need all 1024 / K rows' accumulators at once); its table
  // holds W itself
  constexpr bool V1 = K1 <= 8, V2 = K2E <= 8;
  constexpr int LK2 = K2E == 8 ? 3 : K2E == 4 ? 2 : 1;  // log2(K2) for a vector-ALU middle phase
  constexpr int NMID = K3 ? kFuseMaxChain - 2 : 1;      // the most middle steps
  constexpr int BT1 = V1 ? 2 * K1 * K1 : (K1 == 32 ? 2 : 1) * K1 * 64;
  // a chain's middle tables sit 64 complex entries apart (K <= 8)
  constexpr int BT2 = K3 ? (kFuseMaxChain - 2) * 128 : V2 ? 2 * K2 * K2 : (K2 == 32 ? 2 : 1) * K2 * 64;
  constexpr int BT3 = K3 ? 2 * K3 * K3 : 2;
  // chains of three or more run every phase on the vector ALU
  static_assert(K3 == 0 || (V1 && V2 && K3 <= 8), "chains of three or more have K <= 8");
  static_assert((1 << LB1) == ROWS1 && 8 * WB < 65536, "fused block layout");
  static_assert(kFuseMaxOuter % 6 == 0, "pass-index chunks");
  __shared__ float4 buf[4][WB];
  __shared__ float bt1[BT1], bt2[BT2], bt3[BT3];
  __shared__ int64_t rowoff[ROWSL], coloff[KL];
  __shared__ int64_t ochunk[kFuseMaxOuter / 6][64];  // round-index offsets, 6 bits per chunk
  __shared__ int32_t bit_of[12];
  __shared__ int32_t pairs_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;

  if constexpr (V1) {
    for (int e = tid; e < K1 * K1; e += 256) *(float2 *)&bt1[2 * e] = a.W[0][e];
  } else {
    fused_btable<K1>(a.W[0], bt1, tid);
  }
  if constexpr (V2) {
    if constexpr (K3 != 0) {
      // the chain's middle steps' tables, 64 complex entries apart (each K <= 8)
      for (int e = tid; e < (a.nsteps - 2) * 64; e += 256) {
        const int m = e >> 6, j = e & 63;
        if (j < a.kmid[m] * a.kmid[m]) *(float2 *)&bt2[2 * e] = a.W[1 + m][j];
      }
    } else {
      for (int e = tid; e < K2 * K2; e += 256) *(float2 *)&bt2[2 * e] = a.W[1][e];
    }
  } else {
    fused_btable<K2>(a.W[1], bt2, tid);
  }
  if constexpr (K3 != 0)
    for (int e = tid; e < K3 * K3; e += 256) *(float2 *)&bt3[2 * e] = a.W[a.nsteps - 1][e];
  for (int t = tid; t < ROWSL + KL; t += 256) {
    int64_t o = 0;
    if (t < ROWSL) {
#pragma unroll
      for (int e = 0; e < LB2; ++e)
        if ((t >> e) & 1) o += a.out_row[e];
      rowoff[t] = o;
    } else {
      const int j = t - ROWSL;
#pragma unroll
      for (int c = 0; c < JB2; ++c)
        if ((j >> c) & 1) o += a.out_col[c];
      coloff[j] = o;
    }
  }
  // a round's pass index is 4 round + wave: its bits 2 .. come from the round
  for (int t = tid; t < kFuseMaxOuter / 6 * 64; t += 256) {
    const int c = t >> 6, v = t & 63;
    int64_t o = 0;
#pragma unroll
    for (int q = 2; q < kFuseMaxOuter; ++q)
      if (((q - 2) / 6) == c && ((v >> ((q - 2) % 6)) & 1) && q < a.nouter) o += a.out_pass[q];
    ochunk[c][v] = o;
  }
  __syncthreads();
  if (tid == 0) {
    // the round's entry bits (columns 0 .. JB2-1, rows JB2 .. 9, wave 10, 11) ordered by stride
    int64_t st[12];
    int pb[12];
    for (int c = 0; c < JB2; ++c) {
      st[c] = coloff[1 << c];
      pb[c] = c;
    }
    for (int e = 0; e < LB2; ++e) {
      st[JB2 + e] = rowoff[1 << e];
      pb[JB2 + e] = JB2 + e;
    }
    st[10] = a.out_pass[0];
    pb[10] = 10;
    st[11] = a.out_pass[1];
    pb[11] = 11;
    for (int i = 1; i < 12; ++i)
      for (int q = i; q > 0 && st[q] < st[q - 1]; --q) {
        const int64_t ts = st[q];
        st[q] = st[q - 1];
        st[q - 1] = ts;
        const int tp = pb[q];
        pb[q] = pb[q - 1];
        pb[q - 1] = tp;
      }
    for (int i = 0; i < 12; ++i) bit_of[i] = pb[i];
    pairs_s = st[0] == 1;
  }
  __syncthreads();
  // The workgroup stores its four passes together, in address order: thread
  // tid's pair i is entries 2 (tid + 256 i), +1 of that order, the same in
  // every round.  Its staged indices (wave w's block at 2 WB w complex
  // entries) and offset within the round are kept in registers.
  auto place = [&](int e, int *idx, int64_t *off) {
    int p = 0;
#pragma unroll
    for (int i = 0; i < 12; ++i)
      if ((e >> i) & 1) p |= 1 << bit_of[i];
    const int w = p >> 10, t = (p >> JB2) & (ROWSL - 1), c = p & (KL - 1);
    *idx = w * 2 * WB + t * SP + c;
    *off = rowoff[t] + coloff[c] + ((w & 1) ? a.out_pass[0] : 0) + ((w & 2) ? a.out_pass[1] : 0);
  };
  int32_t sidx[NPT];
  int64_t soff[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    int i0, i1;
    int64_t o1;
    place(2 * (tid + 256 * i), &i0, &soff[i]);
    place(2 * (tid + 256 * i) + 1, &i1, &o1);
    sidx[i] = i0 | (i1 << 16);
  }

  // place of a phase-1 product in the phase-2 block: lane part (its column
  // and the row bit h) plus the row bits fixed by (nb, r)
  const int j1 = K1 == 32 ? l32 : (l32 & 15);
  const int32_t *prow0 = a.pos_row[0], *pcol0 = a.pos_col[0];
  int lane_pos = h ? prow0[2] : 0;
#pragma unroll
  for (int c = 0; c < (K1 == 32 ? 5 : 4); ++c)
    if ((j1 >> c) & 1) lane_pos += pcol0[c];
  auto rpos = [&](int nb, int r) {
    int p = 0;
    if (r & 1) p += prow0[0];
    if (r & 2) p += prow0[1];
    if (r & 4) p += prow0[3];
    if (r & 8) p += prow0[4];
    if (nb & 1) p += prow0[5];
    return p;
  };
  // vector-ALU phases: lane l takes block rows l + 64 i; the lane's row bits
  // (0 .. 5) place its products, bits 6 .. 8 come from i
  int lane_pos_v = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b)
    if ((lane >> b) & 1) lane_pos_v += prow0[b];

  const bool pairs = pairs_s && aligned16(a.C);
  const int64_t nround = (a.R / ROWS1) >> 2;
  // 16-byte entries as a vector type: values, not structs copied through memory
  const f32x4 *X4 = (const f32x4 *)a.X;
  float4 *xb = buf[wave];
  f32x4 *xv = (f32x4 *)xb;
  float *xf = (float *)xb;
  const float2 *cw = (const float2 *)&buf[0][0];
  f32x4 ld[LPT];
  // lane l's load i reads entry pair l % (K1 / 2) of pass row rho = l / (K1 / 2)
  // + i 64 / (K1 / 2); a pass row's X row spreads rho's bits over lrow
  auto spread = [&](int rho) {
    int64_t v = 0;
#pragma unroll
    for (int j = 0; j < LB1; ++j)
      if ((rho >> j) & 1) v += int64_t(1) << a.lrow[j];
    return v;
  };
  const int64_t lane_row = spread(lane >> LKH) + (((int64_t)(wave & 1)) << a.wbit[0]) +
                           (((int64_t)(wave >> 1)) << a.wbit[1]);
  auto load = [&](int64_t rnd) {
    // the round's first X row: its index with zeros put in at the local and wave bits
    uint64_t v = (uint64_t)rnd;
#pragma unroll
    for (int j = 0; j < LB1 + 2; ++j) {
      const int p = a.hole[j];
      v = ((v >> p) << (p + 1)) | (v & ((uint64_t(1) << p) - 1));
    }
    const f32x4 *src = X4 + ((int64_t)v + lane_row) * (K1 / 2) + (lane & (K1 / 2 - 1));
#pragma unroll
    for (int i = 0; i < LPT; ++i) ld[i] = src[spread(i << (6 - LKH)) * (K1 / 2)];
  };
  int64_t rnd = blockIdx.x;
  if (rnd < nround) load(rnd);
  for (; rnd < nround; rnd += gridDim.x) {
    // every wave has finished the last round's stores from the blocks
    __syncthreads();
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int g = lane + 64 * i;
      xv[(g / (K1 / 2)) * RS1 + g % (K1 / 2)] = ld[i];
    }
    if (rnd + gridDim.x < nround) load(rnd + gridDim.x);
    {
      // vector-ALU phases: lane l takes block rows l + 64 i.  An opaque zero
      // per pass keeps their W reads (and the lane's places) in the loop
      // instead of in registers across it.
      constexpr int RPL1 = ROWS1 / 64, RPL2 = ROWS2 / 64;
      [[maybe_unused]] float2 *x2 = (float2 *)xb;
      int wo = 0;
      asm volatile("" : "+v"(wo));
      [[maybe_unused]] const float2 *w1 = (const float2 *)bt1 + wo, *w2 = (const float2 *)bt2 + wo;
      [[maybe_unused]] const float2 *w3 = (const float2 *)bt3 + wo;
      if constexpr (V1) {
        // every read of the block comes before the first write (in place)
        float2 x[RPL1][K1];
#pragma unroll
        for (int i = 0; i < RPL1; ++i)
#pragma unroll
          for (int q = 0; q < K1 / 2; ++q) {
            const float4 f = xb[(lane + 64 * i) * RS1 + q];
            x[i][2 * q] = make_float2(f.x, f.y);
            x[i][2 * q + 1] = make_float2(f.z, f.w);
          }
        const int lp = lane_pos_v + wo;
#pragma unroll
        for (int s2 = 0; s2 < K1; ++s2) {
          float2 w[K1];
#pragma unroll
          for (int k = 0; k < K1; ++k) w[k] = w1[s2 * K1 + k];
          int pc = 0;
#pragma unroll
          for (int c = 0; c < LKH + 1; ++c)
            if ((s2 >> c) & 1) pc += pcol0[c];
#pragma unroll
          for (int i = 0; i < RPL1; ++i) {
            float2 y = make_float2(0.f, 0.f);
#pragma unroll
            for (int k = 0; k < K1; ++k) {
              y.x += x[i][k].x * w[k].x - x[i][k].y * w[k].y;
              y.y += x[i][k].x * w[k].y + x[i][k].y * w[k].x;
            }
            x2[lp + fused_rowhi(prow0, i) + pc] = y;
          }
        }
      } else {
        f32x16 acc[NB1], acw[NB1];
        fused_phase<K1, NB1>(xb, bt1, lane, acc, acw);
        // the lane's base place, opaque per pass so that its 16 NB1 sums with
        // the (uniform) row parts are formed here rather than held in registers
        int lp = lane_pos;
        asm volatile("" : "+v"(lp));
        if constexpr (K1 == 32) {
#pragma unroll
          for (int nb = 0; nb < NB1; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              *(float2 *)&xf[2 * (lp + rpos(nb, r))] = make_float2(acc[nb][r], acw[nb][r]);
        } else {
          const int part = l32 >> 4;
#pragma unroll
          for (int nb = 0; nb < NB1; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) xf[2 * (lp + rpos(nb, r)) + part] = acc[nb][r];
        }
      }
      if constexpr (K3 != 0 && K2 == 0) {
        // the chain's middle steps, each with its own K, table and places
        // in the next step's block
#pragma unroll
        for (int m = 0; m < kFuseMaxChain - 2; ++m) {
          if (m >= a.nsteps - 2) break;
          const float2 *wm = w2 + m * 64;
          const int32_t *prow = a.pos_row[1 + m], *pcol = a.pos_col[1 + m];
          if (a.kmid[m] == 2) fused_mid_step<2>(xb, x2, wm, lane, wo, prow, pcol);
          else if (a.kmid[m] == 4) fused_mid_step<4>(xb, x2, wm, lane, wo, prow, pcol);
          else fused_mid_step<8>(xb, x2, wm, lane, wo, prow, pcol);
        }
      } else if constexpr (V2) {
        // the second step, and in a chain whose middle steps share K2 every
        // step up to the last, each with its own table and places in the
        // next step's block
        const int nmid = K3 ? a.nsteps - 2 : 1;
#pragma unroll
        for (int m = 0; m < NMID; ++m) {
          if (m >= nmid) break;
          float2 z[RPL2][K2];
#pragma unroll
          for (int i = 0; i < RPL2; ++i)
#pragma unroll
            for (int q = 0; q < K2 / 2; ++q) {
              const float4 f = xb[(lane + 64 * i) * RS2 + q];
              z[i][2 * q] = make_float2(f.x, f.y);
              z[i][2 * q + 1] = make_float2(f.z, f.w);
            }
          [[maybe_unused]] const int32_t *prow = a.pos_row[1 + m], *pcol = a.pos_col[1 + m];
          [[maybe_unused]] int lp2 = wo;
          if constexpr (K3 != 0) {
#pragma unroll
            for (int b = 0; b < 6; ++b)
              if ((lane >> b) & 1) lp2 += prow[b];
          }
#pragma unroll
          for (int s2 = 0; s2 < K2; ++s2) {
            float2 w[K2];
#pragma unroll
            for (int k = 0; k < K2; ++k) w[k] = w2[m * 64 + s2 * K2 + k];
            int pc = 0;
            if constexpr (K3 != 0) {
#pragma unroll
              for (int c = 0; c < LK2; ++c)
                if ((s2 >> c) & 1) pc += pcol[c];
            }
#pragma unroll
            for (int i = 0; i < RPL2; ++i) {
              float2 y = make_float2(0.f, 0.f);
#pragma unroll
              for (int k = 0; k < K2; ++k) {
                y.x += z[i][k].x * w[k].x - z[i][k].y * w[k].y;
                y.y += z[i][k].x * w[k].y + z[i][k].y * w[k].x;
              }
              if constexpr (K3 != 0)  // to its place in the next step's block
                x2[lp2 + fused_rowhi(prow, i) + pc] = y;
              else
                x2[(lane + 64 * i) * SP + s2 + wo] = y;
            }
          }
        }
      } else {
        f32x16 acc[NB2], acw[NB2];
        fused_phase<K2, NB2>(xb, bt2, lane, acc, acw);
        if constexpr (K2 == 32) {
#pragma unroll
          for (int nb = 0; nb < NB2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              *(float2 *)&xf[((nb * 32 + (r / 4) * 8 + h * 4 + (r % 4)) * SP + l32) * 2] =
                  make_float2(acc[nb][r], acw[nb][r]);
        } else {
          const int j = l32 & 15, part = l32 >> 4;
#pragma unroll
          for (int nb = 0; nb < NB2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              xf[((nb * 32 + (r / 4) * 8 + h * 4 + (r % 4)) * SP + j) * 2 + part] = acc[nb][r];
        }
      }
      if constexpr (K3 != 0) {
        // third phase: the block's rows times W3, staged
        constexpr int RPL3 = ROWS3 / 64;
        float2 z[RPL3][K3];
#pragma unroll
        for (int i = 0; i < RPL3; ++i)
#pragma unroll
          for (int q = 0; q < K3 / 2; ++q) {
            const float4 f = xb[(lane + 64 * i) * RS3 + q];
            z[i][2 * q] = make_float2(f.x, f.y);
            z[i][2 * q + 1] = make_float2(f.z, f.w);
          }
#pragma unroll
        for (int s3 = 0; s3 < K3; ++s3) {
          float2 w[K3];
#pragma unroll
          for (int k = 0; k < K3; ++k) w[k] = w3[s3 * K3 + k];
#pragma unroll
          for (int i = 0; i < RPL3; ++i) {
            float2 y = make_float2(0.f, 0.f);
#pragma unroll
            for (int k = 0; k < K3; ++k) {
              y.x += z[i][k].x * w[k].x - z[i][k].y * w[k].y;
              y.y += z[i][k].x * w[k].y + z[i][k].y * w[k].x;
            }
            x2[(lane + 64 * i) * SP + s3 + wo] = y;
          }
        }
      }
    }
    int64_t base = 0;
#pragma unroll
    for (int c = 0; c < kFuseMaxOuter / 6; ++c) base += ochunk[c][(rnd >> (6 * c)) & 63];
    // the four passes' products are staged
    __syncthreads();
    if (pairs) {
      float2 v0[NPT], v1[NPT];
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        v0[i] = cw[sidx[i] & 0xffff];
        v1[i] = cw[sidx[i] >> 16];
      }
#pragma unroll
      for (int i = 0; i < NPT; ++i)
        *(float4 *)(a.C + base + soff[i]) = make_float4(v0[i].x, v0[i].y, v1[i].x, v1[i].y);
    } else {
      for (int e = tid; e < 4 * E; e += 256) {
        int idx;
        int64_t off;
        place(e, &idx, &off);
        a.C[base + off] = cw[idx];
      }
    }
  }
}

// Thin GEMM-class steps: a short side of T = 32 NCB entries (32, 64 or 128)
// against a long side of many rows, K a power of two from 16 to 64.  Such a
// step sits near the ridge of the FP32 roofline (for T = K = 64 about 32
// flop per byte), so the matrix cores and HBM must both stay busy.  The
// short operand W (T x K) is staged once per workgroup in LDS, as entry pairs
// (w[c][2q], w[c][2q + 1]) at [q][c].  Each wave then streams passes of 32
// long-side rows with no barrier: the rows of a pass are loaded with
// coalesced 16-byte loads (K in chunks of up to 32 entries) into a
// wave-private LDS area and multiplied against W (real and imaginary parts
// on two MFMAs per column block, as in k_cgemm); the next chunk's or pass's
// loads are issued before the current chunk's MFMAs.
//
// Each 32 x 32 block of results goes back through the same LDS area and
// out in address order, as in k_skinny_mfma (every run of C has a
// power-of-two size, so an offset is rowoff(r0) + rowoff(t) + coloff(j) and
// a fixed permutation of the block's entries sorts it).  That permutation,
// the LDS index of each lane's entries and their offsets relative to the
// pass and column block are the same for every pass: when the smallest
// stride is one entry (16-byte pairs), each lane computes them once, and a
// pass costs one batch of independent LDS reads and one 16-byte store per
// pair.  Otherwise the entries are stored one at a time.
template <int K, int NCB, int NW>
__global__ __launch_bounds__(64 * NW) void k_thin_mfma(StepArgs a, SkinnyRuns rn) {
  constexpr int KC = K < 32 ? K : 32;          // K entries staged per chunk
  constexpr int NCH = K / KC;
  constexpr int KH = KC / 2;                   // 16-byte entry pairs per staged row
  constexpr int RSX = KH + 1;                  // LDS row stride (16-byte units), one pad
  constexpr int XW = kSmRows * RSX;
  constexpr int CS = 33;                       // result row stride (odd: column walks spread over the banks)
  constexpr int CW = (kSmRows * CS + 1) / 2;   // one 32 x 32 complex result block
  constexpr int WB = XW > CW ? XW : CW;
  constexpr int LPT = kSmRows * KH / 64;       // 16-byte loads per lane per chunk
  constexpr int T = 32 * NCB;
  constexpr int NPR = kSmRows * 32 / 128;      // 16-byte pairs per lane per block
  static_assert(kSmRows * KH % 64 == 0, "chunk loads");
  __shared__ float4 buf[NW][WB];
  __shared__ float4 wsh[(K / 2) * T];
  __shared__ int64_t rowoff[kSmRows], coloff[T];
  __shared__ uint16_t perm[kSmRows * 32];
  __shared__ int32_t bit_of[10];
  __shared__ int32_t pairs_s;
  // per lane (the same for every wave) and pair: the two entries' LDS
  // indices (t * CS + j) and the first entry's offset within its pass and
  // column block
  __shared__ int32_t pidx_s[NPR * 64];
  __shared__ int64_t poff_s[NPR * 64];
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int S = (int)a.S;
  for (int t = tid; t < kSmRows + T; t += NT) {
    if (t < kSmRows) rowoff[t] = run_offset(t, rn.rows, rn.nr);
    else coloff[t - kSmRows] = t - kSmRows < S ? run_offset(t - kSmRows, rn.cols, rn.nc) : 0;
  }
  // W as entry pairs (w[c][2q], w[c][2q + 1]) at [q][c]
  for (int e = tid; e < (K / 2) * T; e += NT) {
    const int q = e / T, c = e % T;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < S) {
      const float2 w0 = a.Y[(int64_t)c * K + 2 * q], w1 = a.Y[(int64_t)c * K + 2 * q + 1];
      v = make_float4(w0.x, w0.y, w1.x, w1.y);
    }
    wsh[e] = v;
  }
  __syncthreads();
  if (tid == 0) {
    // bits 0-4 of a permutation entry are its column in a 32-wide block, bits 5-9 its row
    int64_t st[10];
    int pb[10];
    for (int b = 0; b < 5; ++b) {
      st[b] = coloff[1 << b];
      pb[b] = b;
      st[5 + b] = rowoff[1 << b];
      pb[5 + b] = 5 + b;
    }
    for (int i = 1; i < 10; ++i)
      for (int q = i; q > 0 && st[q] < st[q - 1]; --q) {
        const int64_t ts = st[q];
        st[q] = st[q - 1];
        st[q - 1] = ts;
        const int tp = pb[q];
        pb[q] = pb[q - 1];
        pb[q - 1] = tp;
      }
    for (int i = 0; i < 10; ++i) bit_of[i] = pb[i];
    pairs_s = st[0] == 1;
  }
  __syncthreads();
  for (int e = tid; e < kSmRows * 32; e += NT) {
    int p = 0;
    for (int i = 0; i < 10; ++i)
      if ((e >> i) & 1) p |= 1 << bit_of[i];
    perm[e] = (uint16_t)p;
  }
  __syncthreads();
  for (int q = tid; q < NPR * 64; q += NT) {
    const int e = 2 * (q % 64) + 128 * (q / 64);
    const int p0 = perm[e], p1 = perm[e + 1];
    pidx_s[q] = ((p0 >> 5) * CS + (p0 & 31)) | (((p1 >> 5) * CS + (p1 & 31)) << 16);
    poff_s[q] = rowoff[p0 >> 5] + coloff[p0 & 31];
  }
  __syncthreads();
  // every other stride is then a multiple of two, so a pair's first offset is even
  const bool pairs = pairs_s && aligned16(a.C);
  const int64_t R = a.R, npass = (R + kSmRows - 1) / kSmRows;
  const int64_t wstride = (int64_t)gridDim.x * NW;
  const float4 *X4 = (const float4 *)a.X;
  float4 *xb = buf[wave];
  float4 ld[LPT];
  auto load = [&](int64_t b, int ch) {
    if ((b + 1) * kSmRows <= R) {
      // a full pass: no bounds checks
      const float4 *src = X4 + b * kSmRows * (K / 2) + ch * KH;
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int g = lane + 64 * i;
        ld[i] = src[(g / KH) * (K / 2) + g % KH];
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int g = lane + 64 * i;
      const int64_t row = b * kSmRows + g / KH;
      ld[i] = row < R ? X4[row * (K / 2) + ch * KH + g % KH] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  int64_t blk = (int64_t)blockIdx.x * NW + wave;
  if (blk < npass) load(blk, 0);
  for (; blk < npass; blk += wstride) {
    f32x16 accR[NCB], accI[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        accR[cb][r] = 0.f;
        accI[cb][r] = 0.f;
      }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int g = lane + 64 * i;
        xb[(g / KH) * RSX + g % KH] = ld[i];
      }
      if (ch + 1 < NCH) load(blk, ch + 1);
      else if (blk + wstride < npass) load(blk + wstride, 0);
#pragma unroll
      for (int q = 0; q < KH; ++q) {
        const float4 f = xb[l32 * RSX + q];
        const float x0 = h ? f.y : f.x, x1 = h ? f.w : f.z;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const float4 w = wsh[(ch * KH + q) * T + cb * 32 + l32];
          // real part: (wr, -wi) on the (re, im) K slots; imaginary part: (wi, wr)
          const float r0 = h ? -w.y : w.x, i0 = h ? w.x : w.y, r1 = h ? -w.w : w.z, i1 = h ? w.z : w.w;
          accR[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, r0, accR[cb], 0, 0, 0);
          accI[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, i0, accI[cb], 0, 0, 0);
          accR[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, r1, accR[cb], 0, 0, 0);
          accI[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, i1, accI[cb], 0, 0, 0);
        }
      }
    }
    const int64_t p0 = blk * kSmRows;
    const int64_t base = run_offset(p0, rn.rows, rn.nr);
    const int rows = (int)(R - p0 < kSmRows ? R - p0 : kSmRows);
    float *cf = (float *)xb;
    const float2 *cv = (const float2 *)xb;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *(float2 *)&cf[(((r / 4) * 8 + h * 4 + (r % 4)) * CS + l32) * 2] = make_float2(accR[cb][r], accI[cb][r]);
      float2 *cc = a.C + base + coloff[cb * 32];
      if (pairs && rows == kSmRows) {
        float2 v0[NPR], v1[NPR];
        int64_t off[NPR];
#pragma unroll
        for (int i = 0; i < NPR; ++i) {
          const int32_t pi = pidx_s[i * 64 + lane];
          off[i] = poff_s[i * 64 + lane];
          v0[i] = cv[pi & 0xffff];  // t * CS + j
          v1[i] = cv[pi >> 16];
        }
#pragma unroll
        for (int i = 0; i < NPR; ++i) {
          float4 v = make_float4(v0[i].x, v0[i].y, v1[i].x, v1[i].y);
          float4 *dst = (float4 *)(cc + off[i]);
          if (a.beta) {
            const float4 o = *dst;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *dst = v;
        }
      } else {
        const int64_t *co = coloff + cb * 32;
        for (int e = lane; e < kSmRows * 32; e += 64) {
          const int p = perm[e];
          const int t = p >> 5, j = p & 31;
          if (t < rows) store_c(a.C + base + rowoff[t] + co[j], cv[t * CS + j], a.beta);
        }
      }
    }
  }
}

// K-reduction steps: both output sides at most 32 (R, S <= 32) and a long K
// split into `splits` chunks, as in the closing steps of amplitude trees
// (32 x 32 x 2^25, 4 x 4 x 2^30).  One workgroup per K chunk computes the
// whole R x S partial product of its chunk, reading each operand row once
// with coalesced 16-byte loads, and writes it to the split-K scratch
// [splits, R, S]; k_split_reduce then sums the chunks into C.  (The tiled
// GEMM kernel ran such steps with 7/8 of its 256-row tile empty, and the
// skinny row kernel re-read the second operand once per row.)
//
// Matrix-core form: each wave takes 32-entry sub-chunks of K in turn,
// stages both operands' rows through a wave-private LDS area and
// accumulates the 32 x 32 block (rows or columns beyond R or S are zero)
// with the (re, im) K-slot scheme of k_cgemm; the waves' blocks are summed
// through LDS at the end.
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_kred_mfma(StepArgs a, int64_t kchunk) {
  constexpr int KC = 32, KH = KC / 2, RSX = KH + 1, XW = kSmRows * RSX;
  constexpr int LPT = kSmRows * KH / 64;       // 16-byte loads per lane and operand
  __shared__ float4 buf[NW][2 * XW];           // staged X rows, then Y rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int R = (int)a.R, S = (int)a.S;
  const int64_t K = a.K, KH2 = a.K / 2;
  const int64_t k0 = (int64_t)blockIdx.x * kchunk, k1 = k0 + kchunk < K ? k0 + kchunk : K;
  const int64_t nsub = k1 > k0 ? (k1 - k0) / KC : 0;
  const float4 *X4 = (const float4 *)a.X, *Y4 = (const float4 *)a.Y;
  float4 *xb = buf[wave], *yb = buf[wave] + XW;
  f32x16 accR, accI;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    accR[r] = 0.f;
    accI[r] = 0.f;
  }
  float4 lx[LPT], ly[LPT];
  auto load = [&](int64_t sub) {
    const int64_t c = (k0 + sub * KC) / 2;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int g = lane + 64 * i, row = g / KH, q = g % KH;
      lx[i] = row < R ? X4[row * KH2 + c + q] : make_float4(0.f, 0.f, 0.f, 0.f);
      ly[i] = row < S ? Y4[row * KH2 + c + q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  int64_t sub = wave;
  if (sub < nsub) load(sub);
  for (; sub < nsub; sub += NW) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int g = lane + 64 * i;
      xb[(g / KH) * RSX + g % KH] = lx[i];
      yb[(g / KH) * RSX + g % KH] = ly[i];
    }
    if (sub + NW < nsub) load(sub + NW);
#pragma unroll
    for (int q = 0; q < KH; ++q) {
      const float4 f = xb[l32 * RSX + q], w = yb[l32 * RSX + q];
      const float x0 = h ? f.y : f.x, x1 = h ? f.w : f.z;
      // real part: (yr, -yi) on the (re, im) K slots; imaginary part: (yi, yr)
      const float r0 = h ? -w.y : w.x, i0 = h ? w.x : w.y, r1 = h ? -w.w : w.z, i1 = h ? w.z : w.w;
      accR = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, r0, accR, 0, 0, 0);
      accI = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, i0, accI, 0, 0, 0);
      accR = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, r1, accR, 0, 0, 0);
      accI = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, i1, accI, 0, 0, 0);
    }
  }
  // this wave's 32 x 32 block into its own LDS area (after its last reads
  // of it: one wave's LDS operations complete in order), then the sum over
  // the waves
  float2 *cv = (float2 *)buf[wave];
#pragma unroll
  for (int r = 0; r < 16; ++r) cv[((r / 4) * 8 + h * 4 + (r % 4)) * 32 + l32] = make_float2(accR[r], accI[r]);
  __syncthreads();
  for (int e = tid; e < R * S; e += 64 * NW) {
    const int i = e / S, j = e - (e / S) * S;
    float2 t = make_float2(0.f, 0.f);
    for (int w = 0; w < NW; ++w) {
      const float2 v = ((const float2 *)buf[w])[i * 32 + j];
      t.x += v.x;
      t.y += v.y;
    }
    a.scratch[(int64_t)blockIdx.x * R * S + e] = t;
  }
}

// Vector-ALU form for R S <= 16 outputs, R >= S (RM x SM covers R x S): each thread
// takes entry pairs of the chunk in turn, with the R + S operand rows read
// as 16-byte pairs (one contiguous kilobyte per row and wave instruction),
// and keeps all R S complex sums in registers; wave shuffles and LDS sum
// them over the workgroup.
template <int RM, int SM>
__global__ __launch_bounds__(256) void k_kred_valu(StepArgs a, int64_t kchunk) {
  const int R = (int)a.R, S = (int)a.S;
  const int64_t K = a.K, KH2 = a.K / 2;
  const int64_t k0 = (int64_t)blockIdx.x * kchunk, k1 = k0 + kchunk < K ? k0 + kchunk : K;
  const float4 *X4 = (const float4 *)a.X, *Y4 = (const float4 *)a.Y;
  float2 acc[RM][SM];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int c = 0; c < SM; ++c) acc[r][c] = make_float2(0.f, 0.f);
  const int64_t pend = k1 > k0 ? k1 / 2 : 0;
#pragma unroll 2
  for (int64_t p = k0 / 2 + threadIdx.x; p < pend; p += 256) {
    float4 x[RM], y[SM];
#pragma unroll
    for (int r = 0; r < RM; ++r) x[r] = r < R ? X4[r * KH2 + p] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int c = 0; c < SM; ++c) y[c] = c < S ? Y4[c * KH2 + p] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
      for (int c = 0; c < SM; ++c) {
        acc[r][c].x += x[r].x * y[c].x - x[r].y * y[c].y + x[r].z * y[c].z - x[r].w * y[c].w;
        acc[r][c].y += x[r].x * y[c].y + x[r].y * y[c].x + x[r].z * y[c].w + x[r].w * y[c].z;
      }
  }
  __shared__ float2 red[4][RM * SM];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int c = 0; c < SM; ++c) {
      float vx = acc[r][c].x, vy = acc[r][c].y;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        vx += __shfl_xor(vx, off);
        vy += __shfl_xor(vy, off);
      }
      if (lane == 0) red[wave][r * SM + c] = make_float2(vx, vy);
    }
  __syncthreads();
  if ((int)threadIdx.x < R * S) {
    const int e = threadIdx.x, i = e / S, j = e - (e / S) * S;
    float2 t = make_float2(0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      t.x += red[w][i * SM + j].x;
      t.y += red[w][i * SM + j].y;
    }
    a.scratch[(int64_t)blockIdx.x * R * S + e] = t;
  }
}

// ---------------------------------------------------------------------------
// measurement probes (not part of a contraction): the device's sustained
// FP32 matrix-core rate and HBM copy rate, the denominators a roofline is
// checked against.

// NCH independent chains of v_mfma_f32_32x32x2_f32 per wave, no memory
// traffic in the loop; each thread writes one sum so the chains stay live.
template <int NCH>
__global__ __launch_bounds__(256) void k_probe_mfma(float *out, int32_t iters) {
  f32x16 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  const float x = 1e-3f * (float)(threadIdx.x & 7), y = 1.0f - 1e-3f * (float)(threadIdx.x & 3);
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(c & 1 ? y : x, c & 2 ? x : y, acc[c], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-stride 16-byte copy of n entries, U loads in flight per thread.
template <int U>
__global__ __launch_bounds__(256) void k_probe_copy(const float4 *src, float4 *dst, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * step < n; i += U * step) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * step];
#pragma unroll
    for (int u = 0; u < U; ++u) dst[i + u * step] = v[u];
  }
  for (; i < n; i += step) dst[i] = src[i];
}

// 16-byte copy with one contiguous chunk of `chunk` entries per workgroup
// (measured faster than grid-stride order here), loads and stores
// nontemporal when NT.
typedef float probe_v4f __attribute__((ext_vector_type(4)));
template <bool NT>
__global__ __launch_bounds__(256) void k_probe_copy_chunk(const float4 *src, float4 *dst, int64_t n, int64_t chunk) {
  const int64_t b0 = (int64_t)blockIdx.x * chunk, b1 = b0 + chunk < n ? b0 + chunk : n;
  const probe_v4f *s = (const probe_v4f *)src;
  probe_v4f *d = (probe_v4f *)dst;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += 1024) {
    probe_v4f v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + 256 * u < b1) v[u] = NT ? __builtin_nontemporal_load(&s[i + 256 * u]) : s[i + 256 * u];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + 256 * u < b1) {
        if (NT) __builtin_nontemporal_store(v[u], &d[i + 256 * u]);
        else d[i + 256 * u] = v[u];
      }
  }
}

// sum split-K partials [splits, R, S] into C through the runs
template <typename T>
__global__ void k_split_reduce(StepArgsT<T> a) {
  const int64_t total = a.R * a.S;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
    T acc = czero<T>();
    for (int sp = 0; sp < a.splits; ++sp) {
      const T v = a.scratch[(int64_t)sp * total + e];
      acc.x += v.x;
      acc.y += v.y;
    }
    const int64_t i = e / a.S, j = e - (e / a.S) * a.S;
    store_c(a.C + run_offset(i, a.runs, a.nrr) + run_offset(j, a.runs + a.nrr, a.ncr), acc, a.beta);
  }
}

// ---------------------------------------------------------------------------
// complex GEMM on FP32 MFMA.
//
// Real view: with x = (xr, xi) and y = (yr, yi),
//   Cr = sum_l xr*yr + xi*(-yi),   Ci = sum_l xr*yi + xi*yr.
// v_mfma_f32_32x32x2_f32 multiplies a 32x2 block by a 2x32 block.  Its
// 2-long reduction axis is used for (re, im) of one complex l: lanes 0-31
// supply xr of rows 0-31 and lanes 32-63 supply xi.  For the real-part
// product the second operand carries (yr, -yi); for the imaginary part
// (yi, yr).  So one complex l costs two MFMAs per 32x32 complex block and
// the operation count is exactly 8 R S K.
//
// LDS holds the X tile and the Y tile de-interleaved as two planes (re, im),
// each [rows][BK + pad]; a lane reads four consecutive l of a plane with one
// 16-byte load.  Lanes 0-31 feed (yr | yi) to the (real | imaginary) MFMA,
// lanes 32-63 feed (-yi | yr): plane h for the real part with its sign
// flipped when h = 1, plane 1 - h for the imaginary part.  Two LDS stages overlap
// the global loads of the next K tile with the MFMAs of the current one.

// Workgroups are persistent: workgroup b takes tiles L = b, b + G, b + 2G, ...
// (G = grid size) and keeps its LDS pipeline running across tile
// boundaries, so the first K chunk of the next tile loads while the last
// chunk of the current tile is multiplied and stored.  Tile order: workgroups
// are dealt to the 8 XCDs round-robin, so L is first permuted to give each
// XCD a contiguous range of tiles, which is then walked in groups of 8 tile
// rows (column by column inside a group); an XCD's resident workgroups thus
// cover a compact square of C and share their A and B slabs in its L2.
constexpr uint32_t kSwizzleRows = 8;

__device__ __forceinline__ void tile_coords(uint32_t L, uint32_t tiles_r, uint32_t tiles_c, uint32_t *tr,
                                            uint32_t *tc) {
  const uint32_t ntiles = tiles_r * tiles_c;
  const uint32_t n8 = ntiles / 8 * 8;
  const uint32_t Lp = L < n8 ? (L % 8) * (n8 / 8) + L / 8 : L;
  const uint32_t group = Lp / (kSwizzleRows * tiles_c);
  const uint32_t first = group * kSwizzleRows;
  const uint32_t gsz = min(tiles_r - first, kSwizzleRows);
  const uint32_t in_g = Lp - group * kSwizzleRows * tiles_c;
  *tr = first + in_g % gsz;
  *tc = in_g / gsz;
}

template <int BM, int BN, int BK, int WM, int WN, int NT>
// Row, column and tile indices are 32-bit: the planner keeps R, S and K of
// GEMM-class steps below 2^31.
__global__ __launch_bounds__(NT, NT / 128) void k_cgemm(StepArgs a, int32_t kchunk, uint32_t tiles_r, uint32_t tiles_c) {
  constexpr int PAD = 4;
  constexpr int LDK = BK + PAD;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int WAVES_C = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NT / 64, "one wave per WM x WN block");
  static_assert(BK % 4 == 0, "BK");
  constexpr int A_PER = BM * BK / NT;
  constexpr int B_PER = BN * BK / NT;
  static_assert(A_PER >= 1 && B_PER >= 1, "tile too small for the workgroup");

  __shared__ float As[2][2][BM][LDK];
  __shared__ float Bs[2][2][BN][LDK];
  __shared__ int64_t rowoff[2][BM];
  __shared__ int64_t coloff[2][BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WAVES_C, wc = wave % WAVES_C;
  const int h = lane >> 5, l32 = lane & 31;
  const int split = blockIdx.y;
  const int32_t R = (int32_t)a.R, S = (int32_t)a.S, K = (int32_t)a.K;
  const int32_t k0 = split * kchunk;
  const int32_t k1 = min(K, k0 + kchunk);
  const int32_t nkt = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;
  const uint32_t G = gridDim.x;
  const uint32_t ntiles = tiles_r * tiles_c;
  const int32_t my_tiles = (blockIdx.x < ntiles) ? (int32_t)((ntiles - blockIdx.x + G - 1) / G) : 0;
  const bool partial = a.splits > 1;

  f32x16 accR[MB][NB], accI[MB][NB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          accR[mb][nb][r] = 0.f;
          accI[mb][nb][r] = 0.f;
        }
      }
  };
  auto origin = [&](int32_t j, int32_t *r0, int32_t *c0) {
    uint32_t tr, tc;
    tile_coords(blockIdx.x + (uint32_t)j * G, tiles_r, tiles_c, &tr, &tc);
    *r0 = (int32_t)(tr * BM);
    *c0 = (int32_t)(tc * BN);
  };
  auto tables = [&](int par, int32_t r0, int32_t c0) {
    if (partial) return;
    for (int t = tid; t < BM; t += NT) rowoff[par][t] = (r0 + t < R) ? run_offset(r0 + t, a.runs, a.nrr) : 0;
    for (int t = tid; t < BN; t += NT) coloff[par][t] = (c0 + t < S) ? run_offset(c0 + t, a.runs + a.nrr, a.ncr) : 0;
  };
  // Paired stores: lanes 2t and 2t + 1 hold columns c and c + 1 of the same
  // rows; they swap one value (DPP quad_perm [1,0,3,2]) so that the even lane
  // writes row q and the odd lane row q + 1, each as one 16-byte pair.  Needs
  // C's innermost run (a column mode) of even extent and unit stride, and C
  // 16-byte aligned; every row and column offset is then even.
  const bool pair_store = !partial && a.ncr > 0 && a.runs[a.nrr + a.ncr - 1].stride == 1 &&
                          (a.runs[a.nrr + a.ncr - 1].size % 2) == 0 && aligned16(a.C);
  const bool odd_lane = (l32 & 1) != 0;
  auto epilogue = [&](int par, int32_t r0, int32_t c0) {
    if (pair_store) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col0 = wc * WN + nb * 32 + (l32 & ~1);
          const int32_t gj0 = c0 + col0;
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const int q = wr * WM + mb * 32 + (r / 4) * 8 + h * 4 + (r % 4);
            const float sr = odd_lane ? accR[mb][nb][r] : accR[mb][nb][r + 1];
            const float si = odd_lane ? accI[mb][nb][r] : accI[mb][nb][r + 1];
            const float pr = dpp_f<0xB1>(sr), pi = dpp_f<0xB1>(si);
            const int row = odd_lane ? q + 1 : q;
            float4 v = odd_lane ? make_float4(pr, pi, accR[mb][nb][r + 1], accI[mb][nb][r + 1])
                                : make_float4(accR[mb][nb][r], accI[mb][nb][r], pr, pi);
            if (r0 + row < R && gj0 < S) {
              float4 *p = (float4 *)(a.C + rowoff[par][row] + coloff[par][col0]);
              if (a.beta) {
                const float4 o = *p;
                v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
              }
              *p = v;
            }
          }
        }
      return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = wc * WN + nb * 32 + l32;
        const int32_t gj = c0 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wr * WM + mb * 32 + (r / 4) * 8 + h * 4 + (r % 4);
          const int32_t gi = r0 + row;
          if (gi < R && gj < S) {
            const float2 v = make_float2(accR[mb][nb][r], accI[mb][nb][r]);
            if (partial) a.scratch[((int64_t)split * R + gi) * S + gj] = v;
            else store_c(a.C + rowoff[par][row] + coloff[par][col], v, a.beta);
          }
        }
      }
  };

  zero_acc();
  if (nkt == 0) {
    // an empty K chunk of a split step: its partial sums are zero
    for (int32_t j = 0; j < my_tiles; ++j) {
      int32_t r0, c0;
      origin(j, &r0, &c0);
      epilogue(0, r0, c0);
    }
    return;
  }

  float2 ra[A_PER], rb[B_PER];
  // 16-byte loads of entry pairs (l, l + 1) and 8-byte LDS writes when K is
  // even (every K chunk then starts and ends on an even entry), the operand
  // is 16-byte aligned and each thread holds an even number of its entries
  // per stage; decided per operand, single entries otherwise
  constexpr bool kPairA = A_PER % 2 == 0, kPairB = B_PER % 2 == 0;
  const bool pairs_a = kPairA && (a.K % 2 == 0) && aligned16(a.X);
  const bool pairs_b = kPairB && (a.K % 2 == 0) && aligned16(a.Y);
  auto gload = [&](int32_t r0, int32_t c0, int32_t kt) {
    const int32_t kb = k0 + kt * BK;
    if (kPairA && pairs_a) {
#pragma unroll
      for (int q = 0; q < A_PER / 2; ++q) {
        const int p = tid + NT * q;
        const int row = p / (BK / 2), l = 2 * (p % (BK / 2));
        const int32_t gi = r0 + row, gl = kb + l;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gi < R && gl < k1) v = *(const float4 *)(a.X + (int64_t)gi * K + gl);
        ra[2 * q] = make_float2(v.x, v.y);
        ra[2 * q + 1] = make_float2(v.z, v.w);
      }
    } else {
#pragma unroll
      for (int q = 0; q < A_PER; ++q) {
        const int e = tid + NT * q;
        const int row = e / BK, l = e % BK;
        const int32_t gi = r0 + row, gl = kb + l;
        ra[q] = (gi < R && gl < k1) ? a.X[(int64_t)gi * K + gl] : make_float2(0.f, 0.f);
      }
    }
    if (kPairB && pairs_b) {
#pragma unroll
      for (int q = 0; q < B_PER / 2; ++q) {
        const int p = tid + NT * q;
        const int col = p / (BK / 2), l = 2 * (p % (BK / 2));
        const int32_t gj = c0 + col, gl = kb + l;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gj < S && gl < k1) v = *(const float4 *)(a.Y + (int64_t)gj * K + gl);
        rb[2 * q] = make_float2(v.x, v.y);
        rb[2 * q + 1] = make_float2(v.z, v.w);
      }
    } else {
#pragma unroll
      for (int q = 0; q < B_PER; ++q) {
        const int e = tid + NT * q;
        const int col = e / BK, l = e % BK;
        const int32_t gj = c0 + col, gl = kb + l;
        rb[q] = (gj < S && gl < k1) ? a.Y[(int64_t)gj * K + gl] : make_float2(0.f, 0.f);
      }
    }
  };
  auto lstore = [&](int st) {
    if (kPairA && pairs_a) {
#pragma unroll
      for (int q = 0; q < A_PER / 2; ++q) {
        const int p = tid + NT * q;
        const int row = p / (BK / 2), l = 2 * (p % (BK / 2));
        *(float2 *)&As[st][0][row][l] = make_float2(ra[2 * q].x, ra[2 * q + 1].x);
        *(float2 *)&As[st][1][row][l] = make_float2(ra[2 * q].y, ra[2 * q + 1].y);
      }
    } else {
#pragma unroll
      for (int q = 0; q < A_PER; ++q) {
        const int e = tid + NT * q;
        const int row = e / BK, l = e % BK;
        As[st][0][row][l] = ra[q].x;
        As[st][1][row][l] = ra[q].y;
      }
    }
    if (kPairB && pairs_b) {
#pragma unroll
      for (int q = 0; q < B_PER / 2; ++q) {
        const int p = tid + NT * q;
        const int col = p / (BK / 2), l = 2 * (p % (BK / 2));
        *(float2 *)&Bs[st][0][col][l] = make_float2(rb[2 * q].x, rb[2 * q + 1].x);
        *(float2 *)&Bs[st][1][col][l] = make_float2(rb[2 * q].y, rb[2 * q + 1].y);
      }
    } else {
#pragma unroll
      for (int q = 0; q < B_PER; ++q) {
        const int e = tid + NT * q;
        const int col = e / BK, l = e % BK;
        Bs[st][0][col][l] = rb[q].x;
        Bs[st][1][col][l] = rb[q].y;
      }
    }
  };

  const int arow = wr * WM + l32;
  const int bcol = wc * WN + l32;
  const float sgn = h ? -1.f : 1.f;  // real-part operand: yr (lanes 0-31), -yi (lanes 32-63)

  const int32_t total = my_tiles * nkt;
  int32_t j = 0, kt = 0;        // tile and K chunk of the current iteration
  int32_t r0 = 0, c0 = 0;
  if (total > 0) {
    origin(0, &r0, &c0);
    gload(r0, c0, 0);
    lstore(0);
    tables(0, r0, c0);
  }
  __syncthreads();
  for (int32_t it = 0; it < total; ++it) {
    const int st = it & 1;
    // the next iteration's chunk, possibly of the next tile
    int32_t jn = j, ktn = kt + 1, nr0 = r0, nc0 = c0;
    if (ktn == nkt) {
      ktn = 0;
      ++jn;
      if (jn < my_tiles) origin(jn, &nr0, &nc0);
    }
    const bool more = it + 1 < total;
    if (more) gload(nr0, nc0, ktn);
#pragma unroll
    for (int l4 = 0; l4 < BK; l4 += 4) {
      f32x4 av[MB], brv[NB], biv[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) av[mb] = *(const f32x4 *)&As[st][h][arow + mb * 32][l4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        brv[nb] = sgn * *(const f32x4 *)&Bs[st][h][bcol + nb * 32][l4];
        biv[nb] = *(const f32x4 *)&Bs[st][1 - h][bcol + nb * 32][l4];
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            accR[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb][kk], brv[nb][kk], accR[mb][nb], 0, 0, 0);
            accI[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb][kk], biv[nb][kk], accI[mb][nb], 0, 0, 0);
          }
    }
    if (kt == nkt - 1) {
      epilogue(j & 1, r0, c0);
      zero_acc();
    }
    if (more) {
      lstore(st ^ 1);
      if (ktn == 0) tables(jn & 1, nr0, nc0);
    }
    __syncthreads();
    j = jn;
    kt = ktn;
    r0 = nr0;
    c0 = nc0;
  }
}

// One tile per workgroup (K chunks above 64).  Same MFMA scheme and LDS double
// buffer as k_cgemm, without the multi-tile loop; the tile comes from the
// same XCD-aware order.  NT threads, one wave per WM x WN block: the
// 128x128, 64x256 and 256x64 tiles run 8 waves of 64x32 (128 VGPRs, four
// waves per SIMD with two workgroups per CU).  Loads run two K stages ahead (two register stages),
// and tiles wholly inside C with a K chunk that is a multiple of BK load
// without bounds checks.
template <int BM, int BN, int BK, int WM, int WN, int NT>
__global__ __launch_bounds__(NT, NT / 128) void k_cgemm_tile(StepArgs a, int64_t kchunk, uint32_t tiles_r,
                                                       uint32_t tiles_c) {
  constexpr int PAD = 4;
  constexpr int LDK = BK + PAD;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int WAVES_C = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NT / 64, "one wave per WM x WN block");
  static_assert(BK % 4 == 0, "BK");
  constexpr int A_PER = BM * BK / NT;
  constexpr int B_PER = BN * BK / NT;
  static_assert(A_PER >= 1 && B_PER >= 1, "tile too small for the workgroup");

  __shared__ float As[2][2][BM][LDK];
  __shared__ float Bs[2][2][BN][LDK];
  __shared__ int64_t rowoff[BM];
  __shared__ int64_t coloff[BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WAVES_C, wc = wave % WAVES_C;
  const int h = lane >> 5, l32 = lane & 31;
  uint32_t tr, tc;
  tile_coords(blockIdx.x, tiles_r, tiles_c, &tr, &tc);
  const int64_t r0 = (int64_t)tr * BM, c0 = (int64_t)tc * BN;
  const int split = blockIdx.y;
  const int64_t k0 = (int64_t)split * kchunk;
  const int64_t k1 = min(a.K, k0 + kchunk);
  const int64_t nkt = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;
  const int64_t R = a.R, S = a.S, K = a.K;

  f32x16 accR[MB][NB], accI[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        accR[mb][nb][r] = 0.f;
        accI[mb][nb][r] = 0.f;
      }
    }

  // two register stages: the loads of K stage kt + 2 are in flight while
  // stage kt + 1 is written to LDS and stage kt is multiplied
  float2 ra[2][A_PER], rb[2][B_PER];
  // single 8-byte entries per load (16-byte pair loads were slower here on
  // the largest shapes); a tile wholly inside C whose K chunk is a multiple
  // of BK loads without bounds checks
  const bool interior = r0 + BM <= R && c0 + BN <= S && (k1 - k0) % BK == 0;
  auto gload = [&](auto bufc, int64_t kt) {
    constexpr int buf = decltype(bufc)::value;
    const int64_t kb = k0 + kt * BK;
    if (interior) {
#pragma unroll
      for (int q = 0; q < A_PER; ++q) {
        const int e = tid + NT * q;
        ra[buf][q] = a.X[(r0 + e / BK) * K + kb + e % BK];
      }
#pragma unroll
      for (int q = 0; q < B_PER; ++q) {
        const int e = tid + NT * q;
        rb[buf][q] = a.Y[(c0 + e / BK) * K + kb + e % BK];
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int e = tid + NT * q;
      const int row = e / BK, l = e % BK;
      const int64_t gi = r0 + row, gl = kb + l;
      ra[buf][q] = (gi < R && gl < k1) ? a.X[gi * K + gl] : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
      const int e = tid + NT * q;
      const int col = e / BK, l = e % BK;
      const int64_t gj = c0 + col, gl = kb + l;
      rb[buf][q] = (gj < S && gl < k1) ? a.Y[gj * K + gl] : make_float2(0.f, 0.f);
    }
  };
  auto lstore = [&](auto bufc, int st) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int e = tid + NT * q;
      const int row = e / BK, l = e % BK;
      As[st][0][row][l] = ra[buf][q].x;
      As[st][1][row][l] = ra[buf][q].y;
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
      const int e = tid + NT * q;
      const int col = e / BK, l = e % BK;
      Bs[st][0][col][l] = rb[buf][q].x;
      Bs[st][1][col][l] = rb[buf][q].y;
    }
  };

  const int arow = wr * WM + l32;
  const int bcol = wc * WN + l32;
  const float sgn = h ? -1.f : 1.f;  // real-part operand: yr (lanes 0-31), -yi (lanes 32-63)

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (nkt > 0) {
    gload(I0{}, 0);
    if (nkt > 1) gload(I1{}, 1);
    lstore(I0{}, 0);
  }
  __syncthreads();
  // one K stage; the register stage and LDS buffer indices are compile-time
  // constants (kt & 1), so the stage loop is unrolled by two
  auto iter = [&](int64_t kt, auto cur) {
    constexpr int st = decltype(cur)::value;
    using Other = std::integral_constant<int, 1 - st>;
    // scheduling hint: interleave the stage's LDS reads with its MFMAs
    // (measured +0.4% on the sweep; the persistent kernel lost with it)
    __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int l4 = 0; l4 < BK; l4 += 4) {
      if (l4 == BK / 2) {
        // stage kt + 1 (loaded one stage ago) into the other LDS buffer, whose
        // readers finished before the last barrier; then the loads of stage
        // kt + 2 into the registers this frees
        if (kt + 1 < nkt) lstore(Other{}, 1 - st);
        if (kt + 2 < nkt) gload(cur, kt + 2);
      }
      f32x4 av[MB], brv[NB], biv[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) av[mb] = *(const f32x4 *)&As[st][h][arow + mb * 32][l4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        brv[nb] = sgn * *(const f32x4 *)&Bs[st][h][bcol + nb * 32][l4];
        biv[nb] = *(const f32x4 *)&Bs[st][1 - h][bcol + nb * 32][l4];
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            accR[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb][kk], brv[nb][kk], accR[mb][nb], 0, 0, 0);
            accI[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb][kk], biv[nb][kk], accI[mb][nb], 0, 0, 0);
          }
    }
    __syncthreads();
  };
  int64_t kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    iter(kt, I0{});
    iter(kt + 1, I1{});
  }
  if (kt < nkt) iter(kt, I0{});

  const bool partial = a.splits > 1;
  if (!partial) {
    for (int t = tid; t < BM; t += NT) rowoff[t] = (r0 + t < R) ? run_offset(r0 + t, a.runs, a.nrr) : 0;
    for (int t = tid; t < BN; t += NT) coloff[t] = (c0 + t < S) ? run_offset(c0 + t, a.runs + a.nrr, a.ncr) : 0;
  }
  __syncthreads();
  // paired 16-byte stores, as in k_cgemm
  const bool pair_store = !partial && a.ncr > 0 && a.runs[a.nrr + a.ncr - 1].stride == 1 &&
                          (a.runs[a.nrr + a.ncr - 1].size % 2) == 0 && aligned16(a.C);
  if (pair_store) {
    const bool odd_lane = (l32 & 1) != 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col0 = wc * WN + nb * 32 + (l32 & ~1);
        const int64_t gj0 = c0 + col0;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int q = wr * WM + mb * 32 + (r / 4) * 8 + h * 4 + (r % 4);
          const float sr = odd_lane ? accR[mb][nb][r] : accR[mb][nb][r + 1];
          const float si = odd_lane ? accI[mb][nb][r] : accI[mb][nb][r + 1];
          const float pr = dpp_f<0xB1>(sr), pi = dpp_f<0xB1>(si);
          const int row = odd_lane ? q + 1 : q;
          float4 v = odd_lane ? make_float4(pr, pi, accR[mb][nb][r + 1], accI[mb][nb][r + 1])
                              : make_float4(accR[mb][nb][r], accI[mb][nb][r], pr, pi);
          if (r0 + row < R && gj0 < S) {
            float4 *p = (float4 *)(a.C + rowoff[row] + coloff[col0]);
            if (a.beta) {
              const float4 o = *p;
              v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
            }
            *p = v;
          }
        }
      }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wc * WN + nb * 32 + l32;
      const int64_t gj = c0 + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * WM + mb * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        const int64_t gi = r0 + row;
        if (gi < R && gj < S) {
          const float2 v = make_float2(accR[mb][nb][r], accI[mb][nb][r]);
          if (partial) a.scratch[((int64_t)split * R + gi) * S + gj] = v;
          else store_c(a.C + rowoff[row] + coloff[col], v, a.beta);
        }
      }
    }
}

// Small GEMM-class steps (R S <= 2^19, K <= 512): too few 128 x 128 tiles
// to occupy the chip, so the tiled kernels wait on one tile's K loop per
// CU.  Here one workgroup of NW waves takes one 32 x 32 block of C and the
// waves split its K range NW ways (chunks of whole 8-entry stages); each
// wave reads its rows of X and Y straight from global memory (the operands
// of a small step sit in L2), one stage ahead, into the (re, im) MFMA scheme
// of k_cgemm; the NW partial blocks are summed through LDS and wave 0
// stores the block (16-byte row pairs when C's innermost run is an even
// unit-stride column run).  Skinny-class steps with fewer than 4096 rows and
// the same bounds run here too.
constexpr int64_t kSmallGemmRS = int64_t(1) << 19;
constexpr int64_t kSmallGemmK = 512;
constexpr int kSmallGemmWaves = 4;

template <bool PAIR, int NW>
__global__ __launch_bounds__(64 * NW) void k_cgemm_small(StepArgs a, uint32_t blocks_c) {
  __shared__ float red[NW - 1][32][64];
  __shared__ int64_t rowoff[32], coloff[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int32_t R = (int32_t)a.R, S = (int32_t)a.S, K = (int32_t)a.K;
  const int32_t r0 = (int32_t)(blockIdx.x / blocks_c) * 32, c0 = (int32_t)(blockIdx.x % blocks_c) * 32;
  if (tid < 32) rowoff[tid] = r0 + tid < R ? run_offset(r0 + tid, a.runs, a.nrr) : 0;
  else if (tid < 64) coloff[tid - 32] = c0 + tid - 32 < S ? run_offset(c0 + tid - 32, a.runs + a.nrr, a.ncr) : 0;

  // this wave's K range, in whole stages of 8 entries
  const int32_t kq = ((K + 8 * NW - 1) / (8 * NW)) * 8;
  const int32_t kb = wave * kq, ke = min(K, kb + kq);
  const int nst = ke > kb ? (ke - kb + 7) / 8 : 0;
  const int32_t row = r0 + l32, col = c0 + l32;
  const bool rv = row < R, cv = col < S;
  const float2 *xrow = a.X + (int64_t)(rv ? row : 0) * K;
  const float2 *yrow = a.Y + (int64_t)(cv ? col : 0) * K;

  f32x16 accR, accI;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    accR[r] = 0.f;
    accI[r] = 0.f;
  }
  // a stage: entries l0 .. l0 + 7 of this lane's X row and Y row
  auto load = [&](float4 (&x)[4], float4 (&y)[4], int st) {
    const int32_t l0 = kb + st * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t l = l0 + 2 * q;
      if constexpr (PAIR) {
        x[q] = rv && l < ke ? *(const float4 *)(xrow + l) : make_float4(0.f, 0.f, 0.f, 0.f);
        y[q] = cv && l < ke ? *(const float4 *)(yrow + l) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        const float2 z = make_float2(0.f, 0.f);
        const float2 x0 = rv && l < ke ? xrow[l] : z, x1 = rv && l + 1 < ke ? xrow[l + 1] : z;
        const float2 y0 = cv && l < ke ? yrow[l] : z, y1 = cv && l + 1 < ke ? yrow[l + 1] : z;
        x[q] = make_float4(x0.x, x0.y, x1.x, x1.y);
        y[q] = make_float4(y0.x, y0.y, y1.x, y1.y);
      }
    }
  };
  auto compute = [&](const float4 (&x)[4], const float4 (&y)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float xa0 = h ? x[q].y : x[q].x, xa1 = h ? x[q].w : x[q].z;
      const float br0 = h ? -y[q].y : y[q].x, bi0 = h ? y[q].x : y[q].y;
      const float br1 = h ? -y[q].w : y[q].z, bi1 = h ? y[q].z : y[q].w;
      accR = __builtin_amdgcn_mfma_f32_32x32x2f32(xa0, br0, accR, 0, 0, 0);
      accI = __builtin_amdgcn_mfma_f32_32x32x2f32(xa0, bi0, accI, 0, 0, 0);
      accR = __builtin_amdgcn_mfma_f32_32x32x2f32(xa1, br1, accR, 0, 0, 0);
      accI = __builtin_amdgcn_mfma_f32_32x32x2f32(xa1, bi1, accI, 0, 0, 0);
    }
  };
  float4 xa[4], ya[4], xb[4], yb[4];
  if (nst > 0) load(xa, ya, 0);
  for (int st = 0; st < nst; st += 2) {
    if (st + 1 < nst) load(xb, yb, st + 1);
    compute(xa, ya);
    if (st + 1 >= nst) break;
    if (st + 2 < nst) load(xa, ya, st + 2);
    compute(xb, yb);
  }

  // sum the waves' blocks in wave 0
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      red[wave - 1][r][lane] = accR[r];
      red[wave - 1][16 + r][lane] = accI[r];
    }
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < NW - 1; ++w)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      accR[r] += red[w][r][lane];
      accI[r] += red[w][16 + r][lane];
    }
  const bool pair_store = a.ncr > 0 && a.runs[a.nrr + a.ncr - 1].stride == 1 &&
                          (a.runs[a.nrr + a.ncr - 1].size % 2) == 0 && aligned16(a.C);
  if (pair_store) {
    const bool odd_lane = (l32 & 1) != 0;
    const int cl0 = l32 & ~1;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int q = (r / 4) * 8 + h * 4 + (r % 4);
      const float sr = odd_lane ? accR[r] : accR[r + 1];
      const float si = odd_lane ? accI[r] : accI[r + 1];
      const float pr = dpp_f<0xB1>(sr), pi = dpp_f<0xB1>(si);
      const int rr = odd_lane ? q + 1 : q;
      float4 v = odd_lane ? make_float4(pr, pi, accR[r + 1], accI[r + 1]) : make_float4(accR[r], accI[r], pr, pi);
      if (r0 + rr < R && c0 + cl0 < S) {
        float4 *p = (float4 *)(a.C + rowoff[rr] + coloff[cl0]);
        if (a.beta) {
          const float4 o = *p;
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *p = v;
      }
    }
    return;
  }
  if (!cv) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int q = (r / 4) * 8 + h * 4 + (r % 4);
    if (r0 + q < R) store_c(a.C + rowoff[q] + coloff[l32], make_float2(accR[r], accI[r]), a.beta);
  }
}

int g_num_cus = 0;

int num_cus() {
  if (g_num_cus <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

template <int BM, int BN, int BK, int WM, int WN>
hipError_t run_cgemm(const StepArgs &a, hipStream_t stream) {
  const int64_t tiles_r = (a.R + BM - 1) / BM, tiles_c = (a.S + BN - 1) / BN;
  int64_t kchunk = a.K;
  if (a.splits > 1) kchunk = ((a.K + a.splits - 1) / a.splits + BK - 1) / BK * BK;
  if (a.R >= (int64_t(1) << 31) || a.S >= (int64_t(1) << 31) || a.K >= (int64_t(1) << 31) ||
      tiles_r * tiles_c >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  // Short K chunks (up to 64): a persistent grid (two workgroups per CU over
  // the K splits, a multiple of 8 so every XCD gets an equal share) hides
  // each tile's load latency behind the previous tile.  Longer K chunks: one
  // tile per workgroup, so co-resident workgroups stay in step through K and
  // share their L2 lines (persistent workgroups drift apart over many
  // tiles), with loads two K stages ahead.
  const int64_t ntiles = tiles_r * tiles_c;
  // eight waves of WM x WN/2 where both tile sides reach 64 (four waves per
  // SIMD at 128 VGPRs); the 32-wide tiles keep four waves (their narrow
  // operand tile has fewer entries per K stage than 512 threads)
  constexpr bool kWide = BM >= 64 && BN >= 64;
  constexpr int TWN = kWide ? WN / 2 : WN, TNT = kWide ? 512 : 256;
  if (kchunk > 64) {
    dim3 grid((unsigned)ntiles, (unsigned)a.splits);
    note_kernel("k_cgemm_tile<%d,%d>", BM, BN);
    hipLaunchKernelGGL((k_cgemm_tile<BM, BN, BK, WM, TWN, TNT>), grid, dim3(TNT), 0, stream, a, kchunk,
                       (uint32_t)tiles_r, (uint32_t)tiles_c);
    return hipGetLastError();
  }
  int64_t g = (2 * (int64_t)num_cus() + a.splits - 1) / a.splits;
  if (g >= 8) g = g / 8 * 8;
  if (g > ntiles) g = ntiles;
  if (g < 1) g = 1;
  dim3 grid((unsigned)g, (unsigned)a.splits);
  note_kernel("k_cgemm<%d,%d>", BM, BN);
  hipLaunchKernelGGL((k_cgemm<BM, BN, BK, WM, TWN, TNT>), grid, dim3(TNT), 0, stream, a, (int32_t)kchunk,
                     (uint32_t)tiles_r, (uint32_t)tiles_c);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// complex64 GEMM in split bf16 (plans with TNC_PREC_BF16X3)
//
// Each FP32 entry x becomes hi = bf16(x) and lo = bf16(x - hi) (round to
// nearest even); a complex entry (re, im) packs into one 32-bit word per
// part (re in the low half).  The product's K axis carries (re, im) as in
// k_cgemm: the first operand's words are used as they are, the second's as
// (yr, -yi) (sign bit of the high half flipped) for the real part and as
// (yi, yr) (halves swapped) for the imaginary part.  Each of the two is
// hi*hi + hi*lo + lo*hi on v_mfma_f32_32x32x16_bf16 (16 K entries = 8
// complex entries per instruction) with FP32 accumulation.  Tiles 128 x 128,
// four waves of 64 x 64, 16 complex entries of K per stage; one LDS buffer
// with the next stage prefetched into registers.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split_complex(float2 v, uint32_t &whi, uint32_t &wlo) {
  const uint32_t rh = bf16_rne(v.x), ih = bf16_rne(v.y);
  const uint32_t rl = bf16_rne(v.x - __uint_as_float(rh << 16));
  const uint32_t il = bf16_rne(v.y - __uint_as_float(ih << 16));
  whi = rh | (ih << 16);
  wlo = rl | (il << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

constexpr int kBf3Tile = 128;
constexpr int kBf3BK = 16;               // complex entries of K per stage
constexpr int kBf3LD = kBf3BK + 4;       // words per LDS row: conflict-free 16-byte reads

__global__ __launch_bounds__(256, 2) void k_cgemm_bf3(StepArgs a, int64_t kchunk, uint32_t tiles_r,
                                                      uint32_t tiles_c) {
  constexpr int BM = kBf3Tile, BN = kBf3Tile, BK = kBf3BK, LD = kBf3LD;
  constexpr int WM = 64, WN = 64, MB = 2, NB = 2, WAVES_C = BN / WN;
  constexpr int PER = BM * BK / 2 / 256;  // entry pairs per thread per operand
  __shared__ uint32_t Xh[BM][LD], Xl[BM][LD], Yh[BN][LD], Yl[BN][LD];
  __shared__ int64_t rowoff[BM], coloff[BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WAVES_C, wc = wave % WAVES_C;
  const int h = lane >> 5, l32 = lane & 31;
  uint32_t tr, tc;
  tile_coords(blockIdx.x, tiles_r, tiles_c, &tr, &tc);
  const int64_t r0 = (int64_t)tr * BM, c0 = (int64_t)tc * BN;
  const int split = blockIdx.y;
  const int64_t k0 = (int64_t)split * kchunk;
  const int64_t k1 = min(a.K, k0 + kchunk);
  const int64_t nkt = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;
  const int64_t R = a.R, S = a.S, K = a.K;
  const bool partial = a.splits > 1;

  if (!partial) {
    for (int t = tid; t < BM; t += 256) rowoff[t] = (r0 + t < R) ? run_offset(r0 + t, a.runs, a.nrr) : 0;
    for (int t = tid; t < BN; t += 256) coloff[t] = (c0 + t < S) ? run_offset(c0 + t, a.runs + a.nrr, a.ncr) : 0;
  }

  f32x16 accR[MB][NB], accI[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        accR[mb][nb][r] = 0.f;
        accI[mb][nb][r] = 0.f;
      }

  // stage registers: entry pairs (l, l + 1) of row p / (BK / 2)
  float2 rx[PER][2], ry[PER][2];
  auto gload = [&](int64_t kt) {
    const int64_t kb = k0 + kt * BK;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int p = tid + 256 * q;
      const int row = p / (BK / 2), l = 2 * (p % (BK / 2));
      const int64_t gi = r0 + row, gj = c0 + row, gl = kb + l;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        rx[q][u] = (gi < R && gl + u < k1) ? a.X[gi * K + gl + u] : make_float2(0.f, 0.f);
        ry[q][u] = (gj < S && gl + u < k1) ? a.Y[gj * K + gl + u] : make_float2(0.f, 0.f);
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int p = tid + 256 * q;
      const int row = p / (BK / 2), l = 2 * (p % (BK / 2));
      uint32_t h0, l0, h1, l1;
      split_complex(rx[q][0], h0, l0);
      split_complex(rx[q][1], h1, l1);
      *(uint2 *)&Xh[row][l] = make_uint2(h0, h1);
      *(uint2 *)&Xl[row][l] = make_uint2(l0, l1);
      split_complex(ry[q][0], h0, l0);
      split_complex(ry[q][1], h1, l1);
      *(uint2 *)&Yh[row][l] = make_uint2(h0, h1);
      *(uint2 *)&Yl[row][l] = make_uint2(l0, l1);
    }
  };

  if (nkt > 0) gload(0);
  for (int64_t kt = 0; kt < nkt; ++kt) {
    __syncthreads();  // the previous stage's fragment reads are done
    lstore();
    __syncthreads();
    if (kt + 1 < nkt) gload(kt + 1);
#pragma unroll
    for (int s2 = 0; s2 < BK / 8; ++s2) {
      const int off = s2 * 8 + h * 4;  // this lane's 4 complex entries (8 K entries) of the step
      bf16x8 ah[MB], al[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        ah[mb] = as_bf16x8(*(const u32x4 *)&Xh[wr * WM + mb * 32 + l32][off]);
        al[mb] = as_bf16x8(*(const u32x4 *)&Xl[wr * WM + mb * 32 + l32][off]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 bh = *(const u32x4 *)&Yh[wc * WN + nb * 32 + l32][off];
        const u32x4 bl = *(const u32x4 *)&Yl[wc * WN + nb * 32 + l32][off];
        const u32x4 sgn = {0x80000000u, 0x80000000u, 0x80000000u, 0x80000000u};
        const bf16x8 brh = as_bf16x8(bh ^ sgn), brl = as_bf16x8(bl ^ sgn);
        const bf16x8 bih = as_bf16x8((bh >> 16) | (bh << 16)), bil = as_bf16x8((bl >> 16) | (bl << 16));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          accR[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], brh, accR[mb][nb], 0, 0, 0);
          accI[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bih, accI[mb][nb], 0, 0, 0);
          accR[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], brl, accR[mb][nb], 0, 0, 0);
          accI[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bil, accI[mb][nb], 0, 0, 0);
          accR[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], brh, accR[mb][nb], 0, 0, 0);
          accI[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bih, accI[mb][nb], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wc * WN + nb * 32 + l32;
      const int64_t gj = c0 + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * WM + mb * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        const int64_t gi = r0 + row;
        if (gi < R && gj < S) {
          const float2 v = make_float2(accR[mb][nb][r], accI[mb][nb][r]);
          if (partial) a.scratch[((int64_t)split * R + gi) * S + gj] = v;
          else store_c(a.C + rowoff[row] + coloff[col], v, a.beta);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// complex128 (FP64) kernels

// Skinny complex128 steps (one side <= 16): one row per thread, each 16-entry
// K chunk of a 256-row tile staged through LDS, the small operand read by
// broadcast, outputs accumulated in registers.
__global__ __launch_bounds__(256) void k_skinny_z(StepArgsZ a, int64_t kchunk) {
  __shared__ double2 xs[256][kRowsKC + 1];
  __shared__ double2 ys[kSkinnyMax][kRowsKC];
  __shared__ int64_t coloff[kSkinnyMax];
  const int tid = threadIdx.x;
  const int S = (int)a.S;
  if (tid < S) coloff[tid] = run_offset(tid, a.runs + a.nrr, a.ncr);
  const int64_t r0 = (int64_t)blockIdx.x * 256;
  const int split = blockIdx.y;
  const int64_t k0 = (int64_t)split * kchunk;
  const int64_t k1 = min(a.K, k0 + kchunk);
  double2 acc[kSkinnyMax];
#pragma unroll
  for (int q = 0; q < kSkinnyMax; ++q) acc[q] = czero<double2>();
  for (int64_t kc = k0; kc < k1; kc += kRowsKC) {
    const int w = (int)min((int64_t)kRowsKC, k1 - kc);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int row = tid / kRowsKC + 16 * p, col = tid % kRowsKC;
      const int64_t gi = r0 + row;
      xs[row][col] = (gi < a.R && col < w) ? a.X[gi * a.K + kc + col] : czero<double2>();
    }
    if (tid < kSkinnyMax * kRowsKC) {
      const int sr = tid / kRowsKC, col = tid % kRowsKC;
      ys[sr][col] = (sr < S && col < w) ? a.Y[(int64_t)sr * a.K + kc + col] : czero<double2>();
    }
    __syncthreads();
    for (int l = 0; l < w; ++l) {
      const double2 x = xs[tid][l];
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S) cmac(acc[q], x, ys[q][l]);
    }
  }
  const int64_t i = r0 + tid;
  if (i < a.R) {
    if (a.splits > 1) {
      double2 *p = a.scratch + ((int64_t)split * a.R + i) * a.S;
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S) p[q] = acc[q];
    } else {
      const int64_t ro = run_offset(i, a.runs, a.nrr);
#pragma unroll
      for (int q = 0; q < kSkinnyMax; ++q)
        if (q < S) store_c(a.C + ro + coloff[q], acc[q], a.beta);
    }
  }
}

// Complex128 GEMM on FP64 MFMA (v_mfma_f64_16x16x4_f64: a 16x4 block times a
// 4x16 block).  Its 4-long reduction axis carries (re, im) of two complex l:
// lanes with k' = lane / 16 in {0, 1, 2, 3} supply x_re(l0), x_im(l0),
// x_re(l1), x_im(l1); the second operand supplies (y_re, -y_im) for the real
// part and (y_im, y_re) for the imaginary part, so two complex l cost two
// MFMAs per 16x16 complex block and the count is exactly 8 m n k flops.
// LDS holds both tiles as (re, im) planes of doubles, [rows][BK + 2]; tiles
// 64x64 (four waves of 32x32), BK = 8, two LDS stages, XCD-aware tile order,
// one tile per workgroup; loads two K stages ahead and unchecked loads for
// interior tiles, as in k_cgemm_tile.
typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256, 2) void k_zgemm(StepArgsZ a, int64_t kchunk, uint32_t tiles_r, uint32_t tiles_c) {
  constexpr int BM = 64, BN = 64, BK = 8, WM = 32, WN = 32;
  constexpr int LDK = BK + 2;
  constexpr int MB = WM / 16, NB = WN / 16;
  constexpr int WAVES_C = BN / WN;
  constexpr int A_PER = BM * BK / 256, B_PER = BN * BK / 256;

  __shared__ double As[2][2][BM][LDK];
  __shared__ double Bs[2][2][BN][LDK];
  __shared__ int64_t rowoff[BM];
  __shared__ int64_t coloff[BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WAVES_C, wc = wave % WAVES_C;
  const int kq = lane >> 4, l16 = lane & 15;
  const int plane = kq & 1, lofs = kq >> 1;
  const double sgn = plane ? -1.0 : 1.0;
  uint32_t tr, tc;
  tile_coords(blockIdx.x, tiles_r, tiles_c, &tr, &tc);
  const int64_t r0 = (int64_t)tr * BM, c0 = (int64_t)tc * BN;
  const int split = blockIdx.y;
  const int64_t k0 = (int64_t)split * kchunk;
  const int64_t k1 = min(a.K, k0 + kchunk);
  const int64_t nkt = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;
  const int64_t R = a.R, S = a.S, K = a.K;

  f64x4 accR[MB][NB], accI[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        accR[mb][nb][r] = 0.0;
        accI[mb][nb][r] = 0.0;
      }

  // two register stages, as in k_cgemm_tile
  double2 ra[2][A_PER], rb[2][B_PER];
  const bool interior = r0 + BM <= R && c0 + BN <= S && (k1 - k0) % BK == 0;
  auto gload = [&](auto bufc, int64_t kt) {
    constexpr int buf = decltype(bufc)::value;
    const int64_t kb = k0 + kt * BK;
    if (interior) {
#pragma unroll
      for (int q = 0; q < A_PER; ++q) {
        const int e = tid + 256 * q;
        ra[buf][q] = a.X[(r0 + e / BK) * K + kb + e % BK];
      }
#pragma unroll
      for (int q = 0; q < B_PER; ++q) {
        const int e = tid + 256 * q;
        rb[buf][q] = a.Y[(c0 + e / BK) * K + kb + e % BK];
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int e = tid + 256 * q;
      const int row = e / BK, l = e % BK;
      const int64_t gi = r0 + row, gl = kb + l;
      ra[buf][q] = (gi < R && gl < k1) ? a.X[gi * K + gl] : czero<double2>();
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
      const int e = tid + 256 * q;
      const int col = e / BK, l = e % BK;
      const int64_t gj = c0 + col, gl = kb + l;
      rb[buf][q] = (gj < S && gl < k1) ? a.Y[gj * K + gl] : czero<double2>();
    }
  };
  auto lstore = [&](auto bufc, int st) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int e = tid + 256 * q;
      const int row = e / BK, l = e % BK;
      As[st][0][row][l] = ra[buf][q].x;
      As[st][1][row][l] = ra[buf][q].y;
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
      const int e = tid + 256 * q;
      const int col = e / BK, l = e % BK;
      Bs[st][0][col][l] = rb[buf][q].x;
      Bs[st][1][col][l] = rb[buf][q].y;
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (nkt > 0) {
    gload(I0{}, 0);
    if (nkt > 1) gload(I1{}, 1);
    lstore(I0{}, 0);
  }
  __syncthreads();
  auto iter = [&](int64_t kt, auto cur) {
    constexpr int st = decltype(cur)::value;
    using Other = std::integral_constant<int, 1 - st>;
#pragma unroll
    for (int l2 = 0; l2 < BK; l2 += 2) {
      if (l2 == BK / 2) {
        // stage kt + 1 into the other LDS buffer, then the loads of kt + 2
        if (kt + 1 < nkt) lstore(Other{}, 1 - st);
        if (kt + 2 < nkt) gload(cur, kt + 2);
      }
      double av[MB], brv[NB], biv[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) av[mb] = As[st][plane][wr * WM + mb * 16 + l16][l2 + lofs];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        brv[nb] = sgn * Bs[st][plane][wc * WN + nb * 16 + l16][l2 + lofs];
        biv[nb] = Bs[st][1 - plane][wc * WN + nb * 16 + l16][l2 + lofs];
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          accR[mb][nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[mb], brv[nb], accR[mb][nb], 0, 0, 0);
          accI[mb][nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[mb], biv[nb], accI[mb][nb], 0, 0, 0);
        }
    }
    __syncthreads();
  };
  int64_t kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    iter(kt, I0{});
    iter(kt + 1, I1{});
  }
  if (kt < nkt) iter(kt, I0{});

  const bool partial = a.splits > 1;
  if (!partial) {
    for (int t = tid; t < BM; t += 256) rowoff[t] = (r0 + t < R) ? run_offset(r0 + t, a.runs, a.nrr) : 0;
    for (int t = tid; t < BN; t += 256) coloff[t] = (c0 + t < S) ? run_offset(c0 + t, a.runs + a.nrr, a.ncr) : 0;
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wc * WN + nb * 16 + l16;
      const int64_t gj = c0 + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // the FP64 16x16x4 result puts row kq + 4r in register r of lane
        // (kq, col) (the FP32 shapes use 4kq + r)
        const int row = wr * WM + mb * 16 + kq + 4 * r;
        const int64_t gi = r0 + row;
        if (gi < R && gj < S) {
          double2 v;
          v.x = accR[mb][nb][r];
          v.y = accI[mb][nb][r];
          if (partial) a.scratch[((int64_t)split * R + gi) * S + gj] = v;
          else store_c(a.C + rowoff[row] + coloff[col], v, a.beta);
        }
      }
    }
}

template <typename T>
hipError_t run_split_reduce(const StepArgsT<T> &a, hipStream_t stream) {
  const int64_t total = a.R * a.S;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  note_append("+k_split_reduce");
  hipLaunchKernelGGL(k_split_reduce<T>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_header(void **ptab, void *arena, void *out, const void *const *leaves, int32_t num_leaves,
                         const void *blob_src, void *blob_dst, uint64_t blob_bytes, hipStream_t stream) {
  const int32_t total = num_leaves + 2;
  const int64_t n16 = (int64_t)(blob_bytes / 16);
  for (int32_t first = 0; first < total; first += kPtrsPerLaunch) {
    PtrChunk c;
    c.first = first;
    c.count = total - first < kPtrsPerLaunch ? total - first : kPtrsPerLaunch;
    for (int i = 0; i < c.count; ++i) {
      int32_t id = first + i;
      c.p[i] = id == 0 ? arena : id == 1 ? out : const_cast<void *>(leaves[id - 2]);
    }
    // the blob rides with the first chunk
    const int64_t words = first == 0 ? n16 : 0;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 64) blocks = 64;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_header, dim3((unsigned)blocks), dim3(256), 0, stream, ptab, c, (const uint4 *)blob_src,
                       (uint4 *)blob_dst, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_copy(const CopyDesc *descs, int32_t count, int64_t max_count, const void *const *ptab,
                       const int64_t *ints, const SliceDigits &digits, int32_t beta, bool z, hipStream_t stream) {
  int64_t blocks = (max_count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  note_kernel("k_copy");
  if (z)
    hipLaunchKernelGGL(k_copy<double2>, dim3((unsigned)blocks, (unsigned)count), dim3(256), 0, stream, descs, ptab,
                       ints, digits, beta);
  else
    hipLaunchKernelGGL(k_copy<float2>, dim3((unsigned)blocks, (unsigned)count), dim3(256), 0, stream, descs, ptab,
                       ints, digits, beta);
  return hipGetLastError();
}

hipError_t launch_copy_tiled(const CopyDesc *desc, int64_t count, const void *const *ptab, const int64_t *ints,
                             const SliceDigits &digits, int32_t beta, bool z, hipStream_t stream) {
  // passes of 2048 (complex128: 1024) entries, grid-stride over at most
  // 2048 workgroups; `count` here is the entry count of the copy
  const int64_t per = z ? 1024 : 2048;
  int64_t blocks = (count + per - 1) / per;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  note_kernel("k_copy_tiled");
  if (z)
    hipLaunchKernelGGL((k_copy_tiled<double2, 1024>), dim3((unsigned)blocks), dim3(256), 0, stream, desc, ptab, ints,
                       digits, beta);
  else
    hipLaunchKernelGGL((k_copy_tiled<float2, 2048>), dim3((unsigned)blocks), dim3(256), 0, stream, desc, ptab, ints,
                       digits, beta);
  return hipGetLastError();
}

hipError_t launch_tiny(const TinyDesc *descs, int32_t count, int64_t max_rs, const void *const *ptab,
                       const RunDev *runs, int32_t beta, bool z, hipStream_t stream) {
  // a group of few large members spreads each over several workgroups (one
  // per 2048 outputs of the largest member, at most 8, at most 256 in all)
  int64_t parts = count > 0 ? 256 / count : 1;
  if (parts > 8) parts = 8;
  if (parts > max_rs / 2048) parts = max_rs / 2048;
  if (parts < 1) parts = 1;
  const dim3 grid((unsigned)(count * parts));
  note_kernel("k_tiny");
  if (z)
    hipLaunchKernelGGL(k_tiny<double2>, grid, dim3(256), 0, stream, descs, ptab, runs, beta, (int)parts);
  else
    hipLaunchKernelGGL(k_tiny<float2>, grid, dim3(256), 0, stream, descs, ptab, runs, beta, (int)parts);
  return hipGetLastError();
}

template <int K, int SP>
static hipError_t run_skinny_flat(const StepArgs &a, hipStream_t stream) {
  constexpr int G = flat_lanes(K, SP), V = K / (2 * G);
  constexpr bool YREG = V * SP <= 16;
  constexpr int U = V <= 2 ? 2 : 1;
  const int64_t per = (int64_t)(256 / G) * U;
  int64_t blocks = (a.R + per - 1) / per;
  const int64_t cap = 16 * (int64_t)num_cus();
  if (blocks > cap) blocks = cap;
  note_kernel("k_skinny_flat<%d,%d,%d,%s,%d>", G, V, SP, YREG ? "true" : "false", U);
  hipLaunchKernelGGL((k_skinny_flat<G, V, SP, YREG, U>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int SP>
static hipError_t run_skinny_flat_k(const StepArgs &a, hipStream_t stream) {
  switch (a.K) {
    case 2: return run_skinny_flat<2, SP>(a, stream);
    case 4: return run_skinny_flat<4, SP>(a, stream);
    case 8: return run_skinny_flat<8, SP>(a, stream);
    case 16: return run_skinny_flat<16, SP>(a, stream);
    case 32: return run_skinny_flat<32, SP>(a, stream);
    case 64: return run_skinny_flat<64, SP>(a, stream);
    case 128: return run_skinny_flat<128, SP>(a, stream);
    default: return run_skinny_flat<256, SP>(a, stream);
  }
}

static bool skinny_flat_ok(const StepArgs &a) {
  const bool pow2k = a.K >= 2 && a.K <= 256 && (a.K & (a.K - 1)) == 0;
  return a.splits == 1 && a.R >= 4096 && pow2k && a.S >= 1 && a.S <= kSkinnyMax && ((uintptr_t)a.X & 15) == 0;
}

bool small_gemm_ok(const StepArgs &a) { return a.R * a.S <= kSmallGemmRS && a.K <= kSmallGemmK; }

// a step on k_skinny_mfma: long side (rows after orientation) >= 4096, short
// side S a power of two <= 32, K a power of two (<= 64; <= 8 when S = 32)
static bool skinny_mfma_shape_ok(int64_t R, int64_t S, int64_t K) {
  const bool pow2s = S >= 1 && S <= 32 && (S & (S - 1)) == 0;
  const bool pow2k = K >= 2 && K <= (S > 16 ? 8 : 64) && (K & (K - 1)) == 0;
  return R >= 4096 && pow2s && pow2k;
}

static bool skinny_mfma_ok(const StepArgs &a) {
  return a.splits == 1 && a.pow2_runs && skinny_mfma_shape_ok(a.R, a.S, a.K) && ((uintptr_t)a.X & 15) == 0;
}

template <int K, int NB, int SW>
static hipError_t run_skinny_mfma_kn(const StepArgs &a, const SkinnyRuns &rn, hipStream_t stream) {
  const int64_t npass = (a.R + kSmRows * NB - 1) / (kSmRows * NB);
  int64_t blocks = (npass + 3) / 4;
  const int64_t cap = 8 * (int64_t)num_cus();
  if (blocks > cap) blocks = cap;
  note_kernel("k_skinny_mfma<%d,%d,%d>", K, NB, SW);
  hipLaunchKernelGGL((k_skinny_mfma<K, NB, SW>), dim3((unsigned)blocks), dim3(256), 0, stream, a, rn);
  return hipGetLastError();
}

// Tile and sub-blocks per wave pass (32 NB rows; NB S <= 32 and the pass's
// entries ROWS S <= 1024):
// - up to 8 outputs with K <= 8: 16 x 16 x 4 MFMA tiles, which need half the
//   accumulator registers and MFMA time per row of the 32-wide tile there;
//   256 rows per pass for K = 2 (S <= 4), else 128;
// - up to 8 outputs with K = 32, 64: 16 x 16 x 4 tiles, one 32-row block;
// - 16 outputs, or K = 16: the 32-wide tile (real and imaginary parts in
//   its two column halves), one 32-row block per pass;
// - 32 outputs (K <= 8): real and imaginary parts on two MFMAs.
template <int K>
static hipError_t run_skinny_mfma_k(const StepArgs &a, const SkinnyRuns &rn, hipStream_t stream) {
  if constexpr (K <= 2)
    if (a.S <= 4) return run_skinny_mfma_kn<K, 8, 8>(a, rn, stream);
  if constexpr (K <= 8) {
    if (a.S <= 8) return run_skinny_mfma_kn<K, 4, 8>(a, rn, stream);
    if (a.S > 16) return run_skinny_mfma_kn<K, 1, 32>(a, rn, stream);
  } else if constexpr (K >= 32) {
    // up to 8 outputs with K = 32, 64: the narrow tile, one 32-row block per
    // pass (measured 15-18% faster at K = 64; at K = 16 the wide tile is)
    if (a.S <= 8) return run_skinny_mfma_kn<K, 1, 8>(a, rn, stream);
  }
  return run_skinny_mfma_kn<K, 1, 16>(a, rn, stream);
}

static hipError_t run_skinny_mfma(const StepArgs &a, const SkinnyRuns &rn, hipStream_t stream) {
  switch (a.K) {
    case 2: return run_skinny_mfma_k<2>(a, rn, stream);
    case 4: return run_skinny_mfma_k<4>(a, rn, stream);
    case 8: return run_skinny_mfma_k<8>(a, rn, stream);
    case 16: return run_skinny_mfma_k<16>(a, rn, stream);
    case 32: return run_skinny_mfma_k<32>(a, rn, stream);
    default: return run_skinny_mfma_k<64>(a, rn, stream);
  }
}

// K-reduction steps (k_kred_*): a split-K step with both output sides at
// most 32 whose K chunks are whole multiples of 32 entries
static bool kred_ok(const StepArgs &a) {
  if (a.splits <= 1 || a.prec != kPrecExact || a.scratch == nullptr) return false;
  if (a.R < 1 || a.S < 1 || a.R > 32 || a.S > 32) return false;
  if (a.K % ((int64_t)a.splits * 32) != 0) return false;
  return ((uintptr_t)a.X & 15) == 0 && ((uintptr_t)a.Y & 15) == 0;
}

template <int RM, int SM>
static hipError_t run_kred_valu_rs(const StepArgs &a, int64_t kchunk, hipStream_t stream) {
  note_kernel("k_kred_valu<%d,%d>", RM, SM);
  hipLaunchKernelGGL((k_kred_valu<RM, SM>), dim3((unsigned)a.splits), dim3(256), 0, stream, a, kchunk);
  return hipGetLastError();
}

static hipError_t run_kred(const StepArgs &a, hipStream_t stream) {
  const int64_t kchunk = a.K / a.splits;
  hipError_t e;
  // skinny-class steps put the longer side on the rows (R >= S)
  if (a.R * a.S <= 16 && a.R >= a.S) {
    if (a.R <= 4) e = run_kred_valu_rs<4, 4>(a, kchunk, stream);
    else if (a.R <= 8) e = run_kred_valu_rs<8, 2>(a, kchunk, stream);
    else e = run_kred_valu_rs<16, 1>(a, kchunk, stream);
  } else {
    note_kernel("k_kred_mfma<%d>", 4);
    hipLaunchKernelGGL((k_kred_mfma<4>), dim3((unsigned)a.splits), dim3(256), 0, stream, a, kchunk);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return run_split_reduce(a, stream);
}

// thin steps on k_thin_mfma: short side 32, 64 or 128, K in {16, 32, 64}
// (K <= 32 for a short side of 128), long side >= 16384
static bool thin_shape_ok(int64_t R, int64_t S, int64_t K) {
  const bool kk = K == 16 || K == 32 || (K == 64 && S <= 64);
  return R >= 16384 && (S == 32 || S == 64 || S == 128) && kk;
}

template <int K, int NCB, int NW>
static hipError_t run_thin_kn(const StepArgs &a, const SkinnyRuns &rn, hipStream_t stream) {
  const int64_t npass = (a.R + kSmRows - 1) / kSmRows;
  int64_t blocks = (npass + NW - 1) / NW;
  // persistent: as many workgroups as fit on the device at once (LDS bound)
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)k_thin_mfma<K, NCB, NW>, 64 * NW, 0) !=
            hipSuccess ||
        n < 1)
      n = 1;
    per_cu = n;
  }
  const int64_t cap = (int64_t)per_cu * num_cus();
  if (blocks > cap) blocks = cap;
  note_kernel("k_thin_mfma<%d,%d,%d>", K, NCB, NW);
  hipLaunchKernelGGL((k_thin_mfma<K, NCB, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, stream, a, rn);
  return hipGetLastError();
}

static hipError_t run_thin(const StepArgs &a, const SkinnyRuns &rn, hipStream_t stream) {
  if (a.S == 32) {
    if (a.K == 16) return run_thin_kn<16, 1, 12>(a, rn, stream);
    if (a.K == 32) return run_thin_kn<32, 1, 12>(a, rn, stream);
    return run_thin_kn<64, 1, 12>(a, rn, stream);
  }
  if (a.S == 64) {
    // twelve waves (three per SIMD; at most 168 VGPRs, up to 146 KB of LDS)
    if (a.K == 16) return run_thin_kn<16, 2, 12>(a, rn, stream);
    if (a.K == 32) return run_thin_kn<32, 2, 12>(a, rn, stream);
    return run_thin_kn<64, 2, 12>(a, rn, stream);
  }
  if (a.K == 16) return run_thin_kn<16, 4, 8>(a, rn, stream);
  return run_thin_kn<32, 4, 8>(a, rn, stream);
}

static bool gemm_as_thin(const StepArgs &a, hipStream_t stream, hipError_t *err) {
  if (a.splits != 1 || !a.pow2_runs || a.prec != kPrecExact) return false;
  const RunDev *rr = a.runs, *cr = a.runs + a.nrr;
  if (thin_shape_ok(a.R, a.S, a.K) && ((uintptr_t)a.X & 15) == 0) {
    *err = run_thin(a, SkinnyRuns{rr, cr, a.nrr, a.ncr}, stream);
    return true;
  }
  if (thin_shape_ok(a.S, a.R, a.K) && ((uintptr_t)a.Y & 15) == 0) {
    StepArgs b = a;
    b.X = a.Y;
    b.Y = a.X;
    b.R = a.S;
    b.S = a.R;
    *err = run_thin(b, SkinnyRuns{cr, rr, a.ncr, a.nrr}, stream);
    return true;
  }
  return false;
}

// The step as given (rows = R) or exchanged (rows = S): the long side must
// be the row side of k_skinny_mfma.
static bool gemm_as_skinny(const StepArgs &a, hipStream_t stream, hipError_t *err) {
  if (a.splits != 1 || !a.pow2_runs || a.prec != kPrecExact) return false;
  const RunDev *rr = a.runs, *cr = a.runs + a.nrr;
  if (skinny_mfma_shape_ok(a.R, a.S, a.K) && ((uintptr_t)a.X & 15) == 0) {
    *err = run_skinny_mfma(a, SkinnyRuns{rr, cr, a.nrr, a.ncr}, stream);
    return true;
  }
  if (skinny_mfma_shape_ok(a.S, a.R, a.K) && ((uintptr_t)a.Y & 15) == 0) {
    StepArgs b = a;
    b.X = a.Y;
    b.Y = a.X;
    b.R = a.S;
    b.S = a.R;
    *err = run_skinny_mfma(b, SkinnyRuns{cr, rr, a.ncr, a.nrr}, stream);
    return true;
  }
  return false;
}

hipError_t run_cgemm_small(const StepArgs &a, hipStream_t stream) {
  const int64_t bc = (a.S + 31) / 32, blocks = ((a.R + 31) / 32) * bc;
  const bool pair = a.K % 2 == 0 && ((uintptr_t)a.X & 15) == 0 && ((uintptr_t)a.Y & 15) == 0;
  constexpr int NW = kSmallGemmWaves;
  note_kernel("k_cgemm_small<%s,%d>", pair ? "true" : "false", NW);
  if (pair)
    hipLaunchKernelGGL((k_cgemm_small<true, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, stream, a, (uint32_t)bc);
  else
    hipLaunchKernelGGL((k_cgemm_small<false, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, stream, a, (uint32_t)bc);
  return hipGetLastError();
}

template <int K1, int K2, int K3 = 0>
static hipError_t run_fused2_k(const Fused2Args &a, hipStream_t stream) {
  const int64_t nround = (a.R / (kFuseEntries / K1)) / 4;  // four passes per workgroup round
  int64_t blocks = nround;
  // up to 8 workgroups per CU; a short launch, whose workgroups would get
  // fewer than 16 rounds each, only those resident at once (two per CU by
  // registers and LDS), so that each amortizes its table set-up over more
  // rounds
  const int64_t cus = num_cus();
  const int64_t cap = nround < 16 * 8 * cus ? 2 * cus : 8 * cus;
  if (blocks > cap) blocks = cap;
  if (K3) note_kernel("k_fused2<%d,%d,%d>", K1, K2, K3);
  else note_kernel("k_fused2<%d,%d>", K1, K2);
  hipLaunchKernelGGL((k_fused2<K1, K2, K3>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fused2(const Fused2Args &a, hipStream_t stream) {
  // the planner emits only chains that meet these; anything else is refused
  auto kok = [](int32_t k) { return k == 2 || k == 4 || k == 8 || k == 16 || k == 32; };
  if (!kok(a.K1) || !kok(a.K2) || a.nouter < 0 || a.nouter > kFuseMaxOuter) return hipErrorInvalidValue;
  if (a.nsteps < 2 || a.nsteps > kFuseMaxChain || (a.nsteps == 2) != (a.K3 == 0)) return hipErrorInvalidValue;
  if (a.K3 != 0 && (a.K1 > 8 || a.K2 > 8 || (a.K3 != 2 && a.K3 != 4 && a.K3 != 8))) return hipErrorInvalidValue;
  // K = 2 pairs only with vector-ALU partners
  if ((a.K1 == 2 && a.K2 > 8) || (a.K2 == 2 && a.K1 > 8)) return hipErrorInvalidValue;
  for (int q = 0; q < a.nsteps; ++q)
    if (!a.W[q]) return hipErrorInvalidValue;
  if (a.nouter < 2 || a.R != ((int64_t)(kFuseEntries / a.K1) << a.nouter) || !a.X || !a.C ||
      ((uintptr_t)a.X & 15) != 0)
    return hipErrorInvalidValue;
  if (a.K3 != 0) {
    // chains of three or more: every K is 2, 4 or 8, the middle ones at run time
    for (int m = 0; m < a.nsteps - 2; ++m)
      if (a.kmid[m] != 2 && a.kmid[m] != 4 && a.kmid[m] != 8) return hipErrorInvalidValue;
    // middle steps that share one K run the instance compiled for it
    bool same = true;
    for (int m = 1; m < a.nsteps - 2; ++m) same = same && a.kmid[m] == a.kmid[0];
    const int k2 = same ? a.kmid[0] : 0;
    auto last = [&](auto k1c, auto k2c) {
      constexpr int k1 = decltype(k1c)::value, kk2 = decltype(k2c)::value;
      switch (a.K3) {
        case 2: return run_fused2_k<k1, kk2, 2>(a, stream);
        case 4: return run_fused2_k<k1, kk2, 4>(a, stream);
        default: return run_fused2_k<k1, kk2, 8>(a, stream);
      }
    };
    auto middle = [&](auto k1c) {
      switch (k2) {
        case 0: return last(k1c, std::integral_constant<int, 0>{});
        case 2: return last(k1c, std::integral_constant<int, 2>{});
        case 4: return last(k1c, std::integral_constant<int, 4>{});
        default: return last(k1c, std::integral_constant<int, 8>{});
      }
    };
    switch (a.K1) {
      case 2: return middle(std::integral_constant<int, 2>{});
      case 4: return middle(std::integral_constant<int, 4>{});
      default: return middle(std::integral_constant<int, 8>{});
    }
  }
  auto second = [&](auto k1c) {
    constexpr int k1 = decltype(k1c)::value;
    if constexpr (k1 == 2) {
      switch (a.K2) {
        case 2: return run_fused2_k<2, 2>(a, stream);
        case 4: return run_fused2_k<2, 4>(a, stream);
        default: return run_fused2_k<2, 8>(a, stream);
      }
    } else {
      switch (a.K2) {
        case 2:
          if constexpr (k1 <= 8) return run_fused2_k<k1, 2>(a, stream);
          else return hipErrorInvalidValue;
        case 4: return run_fused2_k<k1, 4>(a, stream);
        case 8: return run_fused2_k<k1, 8>(a, stream);
        case 16: return run_fused2_k<k1, 16>(a, stream);
        default: return run_fused2_k<k1, 32>(a, stream);
      }
    }
  };
  switch (a.K1) {
    case 2: return second(std::integral_constant<int, 2>{});
    case 4: return second(std::integral_constant<int, 4>{});
    case 8: return second(std::integral_constant<int, 8>{});
    case 16: return second(std::integral_constant<int, 16>{});
    default: return second(std::integral_constant<int, 32>{});
  }
}

hipError_t launch_skinny(const StepArgs &a, hipStream_t stream) {
  if (skinny_mfma_ok(a)) return run_skinny_mfma(a, SkinnyRuns{a.runs, a.runs + a.nrr, a.nrr, a.ncr}, stream);
  if (skinny_flat_ok(a)) {
    if (a.S <= 1) return run_skinny_flat_k<1>(a, stream);
    if (a.S <= 2) return run_skinny_flat_k<2>(a, stream);
    if (a.S <= 4) return run_skinny_flat_k<4>(a, stream);
    if (a.S <= 8) return run_skinny_flat_k<8>(a, stream);
    return run_skinny_flat_k<16>(a, stream);
  }
  // few rows and a short K: the small-GEMM kernel (one workgroup per 32-row
  // block) instead of one workgroup per row
  if (a.R < 4096 && a.splits <= 1 && small_gemm_ok(a)) return run_cgemm_small(a, stream);
  // at most 32 x 32 outputs over a long, split K: one workgroup per K chunk
  if (kred_ok(a)) return run_kred(a, stream);
  int64_t kchunk = a.K;
  if (a.splits > 1) kchunk = (a.K + a.splits - 1) / a.splits;
  // outer products of a long operand (K = 1): streamed by k_outer
  if (a.R >= 4096 && a.splits == 1 && a.K == 1 && a.S <= kSkinnyMax && a.nrr >= 1) {
    int64_t blocks = (a.R / 2 + 256 * kOuterU - 1) / (256 * kOuterU);
    const int64_t cap = 8 * (int64_t)num_cus();
    if (blocks > cap) blocks = cap;
    note_kernel("k_outer");
    hipLaunchKernelGGL(k_outer, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  // kernel choice measured on MI355X: rows of >= 8 entries stream fastest
  // straight into registers; shorter rows are read as one contiguous block
  // per 256 rows through LDS (grid-stride); chunked K one tile per workgroup
  if (a.R >= 4096 && a.splits == 1 && a.K >= 8 && a.K <= kRowsKC) {
    const int rows = a.K <= 8 ? 2 : 1;
    const int64_t blocks = (a.R + 256 * rows - 1) / (256 * rows);
    note_kernel("k_skinny_small<%d>", rows);
    if (rows == 2) hipLaunchKernelGGL(k_skinny_small<2>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_skinny_small<1>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  } else if (a.R >= 4096 && a.splits == 1 && a.K < 8) {
    const int64_t tiles = (a.R + 255) / 256;
    int64_t g = 8 * (int64_t)num_cus();
    if (g > tiles) g = tiles;
    note_kernel("k_skinny_rows");
    hipLaunchKernelGGL(k_skinny_rows, dim3((unsigned)g, 1), dim3(256), 0, stream, a, kchunk);
    return hipGetLastError();
  } else if (a.R >= 4096) {
    // many rows, K in chunks: one tile of 256 rows per workgroup
    const int64_t tiles = (a.R + 255) / 256;
    note_kernel("k_skinny_rows");
    hipLaunchKernelGGL(k_skinny_rows, dim3((unsigned)tiles, (unsigned)a.splits), dim3(256), 0, stream, a, kchunk);
  } else {
    note_kernel("k_skinny");
    hipLaunchKernelGGL(k_skinny, dim3((unsigned)a.R, (unsigned)a.splits), dim3(256), 0, stream, a, kchunk);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  return run_split_reduce(a, stream);
}

hipError_t launch_gemm(const StepArgs &a, hipStream_t stream) {
  if (a.prec == kPrecBf16x3) {
    const int64_t tiles_r = (a.R + kBf3Tile - 1) / kBf3Tile, tiles_c = (a.S + kBf3Tile - 1) / kBf3Tile;
    int64_t kchunk = a.K;
    if (a.splits > 1) kchunk = ((a.K + a.splits - 1) / a.splits + kBf3BK - 1) / kBf3BK * kBf3BK;
    if (tiles_r * tiles_c >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    note_kernel("k_cgemm_bf3");
    hipLaunchKernelGGL(k_cgemm_bf3, dim3((unsigned)(tiles_r * tiles_c), (unsigned)a.splits), dim3(256), 0, stream, a,
                       kchunk, (uint32_t)tiles_r, (uint32_t)tiles_c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits <= 1) return e;
    return run_split_reduce(a, stream);
  }
  // small steps: one workgroup per 32 x 32 block, K split over its waves
  if (small_gemm_ok(a)) return run_cgemm_small(a, stream);
  // a short side of at most 32 with a short K: memory-bound, streamed like a skinny step
  {
    hipError_t e = hipSuccess;
    if (gemm_as_thin(a, stream, &e)) return e;
    if (gemm_as_skinny(a, stream, &e)) return e;
  }
  if (kred_ok(a)) return run_kred(a, stream);
  // tile shape: keep the short side of the step inside one tile edge
  hipError_t e;
  if (a.S > 64 && a.R <= 32) e = run_cgemm<32, 256, 8, 32, 64>(a, stream);
  else if (a.S > 64 && a.R <= 64) e = run_cgemm<64, 256, 8, 64, 64>(a, stream);
  else if (a.S > 64) e = run_cgemm<128, 128, 8, 64, 64>(a, stream);
  else if (a.S > 32) e = run_cgemm<256, 64, 8, 64, 64>(a, stream);
  else e = run_cgemm<256, 32, 8, 64, 32>(a, stream);
  if (e != hipSuccess || a.splits <= 1) return e;
  return run_split_reduce(a, stream);
}

hipError_t launch_skinny_z(const StepArgsZ &a, hipStream_t stream) {
  int64_t kchunk = a.K;
  if (a.splits > 1) kchunk = (a.K + a.splits - 1) / a.splits;
  dim3 grid((unsigned)((a.R + 255) / 256), (unsigned)a.splits);
  note_kernel("k_skinny_z");
  hipLaunchKernelGGL(k_skinny_z, grid, dim3(256), 0, stream, a, kchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  return run_split_reduce(a, stream);
}

hipError_t launch_gemm_z(const StepArgsZ &a, hipStream_t stream) {
  constexpr int64_t BM = 64, BN = 64, BK = 8;
  const int64_t tiles_r = (a.R + BM - 1) / BM, tiles_c = (a.S + BN - 1) / BN;
  if (tiles_r * tiles_c >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  int64_t kchunk = a.K;
  if (a.splits > 1) kchunk = ((a.K + a.splits - 1) / a.splits + BK - 1) / BK * BK;
  dim3 grid((unsigned)(tiles_r * tiles_c), (unsigned)a.splits);
  note_kernel("k_zgemm");
  hipLaunchKernelGGL(k_zgemm, grid, dim3(256), 0, stream, a, kchunk, (uint32_t)tiles_r, (uint32_t)tiles_c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  return run_split_reduce(a, stream);
}

hipError_t launch_probe_mfma(float *out, int64_t blocks, int32_t iters, int32_t chains, hipStream_t stream) {
  if (chains >= 8) hipLaunchKernelGGL(k_probe_mfma<8>, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  else hipLaunchKernelGGL(k_probe_mfma<4>, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, int64_t n16, int32_t pattern, hipStream_t stream) {
  const float4 *s = (const float4 *)src;
  float4 *d = (float4 *)dst;
  if (pattern >= 2) {
    const int64_t chunk = int64_t(1) << 14;
    const int64_t blocks = (n16 + chunk - 1) / chunk;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (pattern == 3)
      hipLaunchKernelGGL(k_probe_copy_chunk<true>, dim3((unsigned)blocks), dim3(256), 0, stream, s, d, n16, chunk);
    else
      hipLaunchKernelGGL(k_probe_copy_chunk<false>, dim3((unsigned)blocks), dim3(256), 0, stream, s, d, n16, chunk);
    return hipGetLastError();
  }
  const int64_t blocks = 8 * (int64_t)num_cus();
  if (pattern == 1)
    hipLaunchKernelGGL(k_probe_copy<4>, dim3((unsigned)blocks), dim3(256), 0, stream, s, d, n16);
  else
    hipLaunchKernelGGL(k_probe_copy<1>, dim3((unsigned)blocks), dim3(256), 0, stream, s, d, n16);
  return hipGetLastError();
}

int32_t device_cus() { return (int32_t)num_cus(); }

}  // namespace tnc

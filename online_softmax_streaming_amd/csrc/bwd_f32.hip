// Attention backward for FP32 inputs, on the vector ALUs.
//
// The same quantities as the matrix-core backward, per head, in natural units
// with lse = m + ln l from the forward's row state (the A1 state of the
// answer-key page, "Compare reasoning after your own attempt", row A1):
//   P  = exp(scale Q K^T - lse) on visible keys, 0 elsewhere
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta),  Delta = rowsum(dO * O)
//   dQ = scale dS K,   dK = scale dS^T Q
// dS is the row-wise softmax vector-Jacobian product of the workshops page's
// I2 ("Intermediate and advanced kernel workshops", softmax backward) with
// y = P and g = dP; <P, dP> = rowsum(dO * O) because O = P V.  Everything
// stays FP32 (nothing is rounded to a narrower type), as in the FP32 forward.
// This path is for FP32 accuracy, not throughput.
//
// Two kernels, ordered on one stream:
//   1. dq (query-stationary): a workgroup owns RPB query rows, TP threads
//      per row (DT = D / TP features each, dot products summed across the
//      TP lanes).  The row's Q, dO and dQ stay in registers; tiles of 32
//      keys of K and V are staged in LDS and read by broadcast.  Before the
//      key loop each row forms Delta and the base-2 lse and writes both for
//      kernel 2.
//   2. dkdv (key-stationary): a workgroup owns RPB keys of one K/V head with
//      their K, V, dK, dV rows in registers; tiles of 32 query rows of Q and
//      dO, with the rows' (lse, Delta), are staged in LDS.  With grouped K/V
//      heads the workgroup walks the query heads of its group in turn, so dK
//      and dV sum over the group without atomics.
// Every output element is written once by one thread; no atomics.
//
// Causal visibility is the forward's: key j is visible to query i iff
// j <= i + (Nk - Nq).  Rows past Nq or keys past Nk are staged as zeros and
// get P = 0 explicitly (ghost keys by the visibility test, ghost query rows
// through lse = +inf); rows with no visible key have l = 0, hence lse = +inf
// and P = 0 everywhere.

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

struct BwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dout;
  const float* m;  // [B*H*Nq], natural units
  const float* l;
  float* dq;
  float* dk;
  float* dv;
  float* stat;  // [B*H*Nq][2]: base-2 lse, Delta (kernel 1 writes, kernel 2 reads)
  int H, Hkv, group;
  int Nq, Nk;
  int nqt;  // workgroups per query head in kernel 1
  int nkt;  // workgroups per K/V head in kernel 2
  float c;  // scale * log2(e)
  float scale;
};

constexpr int kThreads = 128;
constexpr int kTile = 32;  // keys (kernel 1) or query rows (kernel 2) per LDS tile
constexpr float kInf = __builtin_inff();

template <int D>
struct F32Split {
  static constexpr int TP = D > 64 ? 4 : (D > 32 ? 2 : 1);  // threads per row
  static constexpr int DT = D / TP;                          // features per thread
  static constexpr int RPB = kThreads / TP;                  // rows per workgroup
};

// Sum over the TP adjacent lanes that share a row.
template <int TP>
__device__ __forceinline__ float row_sum(float x) {
  if (TP >= 2) x += __shfl_xor(x, 1);
  if (TP >= 4) x += __shfl_xor(x, 2);
  return x;
}

// Stage `kTile` rows starting at r0 of a [rows, D] FP32 matrix into LDS;
// rows at or past `n` are zero.
template <int D>
__device__ __forceinline__ void stage_rows(float* dst, const float* src, int r0, int n) {
  for (int e = threadIdx.x; e < kTile * D / 4; e += kThreads) {
    const int row = e / (D / 4), col = e - row * (D / 4);
    const int r = r0 + row;
    f32x4 x = f32x4{};
    if (r < n) x = *reinterpret_cast<const f32x4*>(src + (int64_t)r * D + col * 4);
    *reinterpret_cast<f32x4*>(dst + row * D + col * 4) = x;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_f32_dq_kernel(BwdF32Args a) {
  constexpr int TP = F32Split<D>::TP, DT = F32Split<D>::DT, RPB = F32Split<D>::RPB;
  __shared__ __attribute__((aligned(16))) float Ks[kTile * D];
  __shared__ __attribute__((aligned(16))) float Vs[kTile * D];

  const int bh = blockIdx.x / a.nqt;
  const int qt = blockIdx.x - bh * a.nqt;
  const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
  const int64_t qbase = (int64_t)bh * Nq * D;
  const float* Kh = a.k + (int64_t)(bh / a.group) * Nk * D;
  const float* Vh = a.v + (int64_t)(bh / a.group) * Nk * D;
  const int tid = threadIdx.x;
  const int part = tid % TP;
  const int i0 = qt * RPB;
  const int qrow = i0 + tid / TP;
  const bool real = qrow < Nq;

  float q[DT], g[DT], dq[DT];
  float dlt = 0.f;
#pragma unroll
  for (int d = 0; d < DT; ++d) {
    const int64_t e = qbase + (int64_t)qrow * D + part * DT + d;
    q[d] = real ? a.q[e] : 0.f;
    g[d] = real ? a.dout[e] : 0.f;
    dlt = __builtin_fmaf(g[d], real ? a.o[e] : 0.f, dlt);
    dq[d] = 0.f;
  }
  const float delta = row_sum<TP>(dlt);  // rowsum(dO * O)
  float lse2 = kInf;                      // ghost rows and rows without keys: P = 0
  if (real) {
    const int64_t row = (int64_t)bh * Nq + qrow;
    const float ll = a.l[row];
    lse2 = ll > 0.f ? __builtin_fmaf(a.m[row], kLog2e, log2f(ll)) : kInf;
    if (part == 0) {
      a.stat[2 * row] = lse2;
      a.stat[2 * row + 1] = delta;
    }
  }

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(i0 + RPB, Nq) + off);
  const int ntiles = kend > 0 ? (kend + kTile - 1) / kTile : 0;
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kTile;
    stage_rows<D>(Ks, Kh, j0, Nk);
    stage_rows<D>(Vs, Vh, j0, Nk);
    __syncthreads();
    for (int jj = 0; jj < kTile; ++jj) {
      const float* kr = Ks + jj * D + part * DT;
      const float* vr = Vs + jj * D + part * DT;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        s = __builtin_fmaf(q[d], kr[d], s);
        dp = __builtin_fmaf(g[d], vr[d], dp);
      }
      s = row_sum<TP>(s);
      dp = row_sum<TP>(dp);
      const int j = j0 + jj;
      const bool vis = j < Nk && (!CAUSAL || j <= qrow + off);
      const float p = vis ? exp2_hw(__builtin_fmaf(s, a.c, -lse2)) : 0.f;
      const float ds = p * (dp - delta);
#pragma unroll
      for (int d = 0; d < DT; ++d) dq[d] = __builtin_fmaf(ds, kr[d], dq[d]);
    }
    __syncthreads();
  }
  if (real) {
#pragma unroll
    for (int d = 0; d < DT; ++d) a.dq[qbase + (int64_t)qrow * D + part * DT + d] = dq[d] * a.scale;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_f32_dkdv_kernel(BwdF32Args a) {
  constexpr int TP = F32Split<D>::TP, DT = F32Split<D>::DT, RPB = F32Split<D>::RPB;
  __shared__ __attribute__((aligned(16))) float Qs[kTile * D];
  __shared__ __attribute__((aligned(16))) float Gs[kTile * D];
  __shared__ float Ss[kTile * 2];

  const int bhk = blockIdx.x / a.nkt;  // b * Hkv + kv head
  const int kt = blockIdx.x - bhk * a.nkt;
  const int b = bhk / a.Hkv, hk = bhk - b * a.Hkv;
  const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
  const int64_t kbase = (int64_t)bhk * Nk * D;
  const int tid = threadIdx.x;
  const int part = tid % TP;
  const int j0 = kt * RPB;
  const int key = j0 + tid / TP;
  const bool real = key < Nk;

  float kk[DT], vv[DT], dk[DT], dv[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) {
    const int64_t e = kbase + (int64_t)key * D + part * DT + d;
    kk[d] = real ? a.k[e] : 0.f;
    vv[d] = real ? a.v[e] : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }

  // Query rows that may see a key of this workgroup: i >= j0 - off.
  const int t_first = CAUSAL ? max(0, j0 - off) / kTile : 0;
  const int ntq = (Nq + kTile - 1) / kTile;
  for (int h = hk * a.group; h < (hk + 1) * a.group; ++h) {
    const int64_t bh = (int64_t)b * a.H + h;
    const float* Qh = a.q + bh * Nq * D;
    const float* Gh = a.dout + bh * Nq * D;
    const float* st = a.stat + 2 * bh * Nq;
    for (int t = t_first; t < ntq; ++t) {
      const int r0 = t * kTile;
      stage_rows<D>(Qs, Qh, r0, Nq);
      stage_rows<D>(Gs, Gh, r0, Nq);
      if (tid < kTile) {
        const int r = r0 + tid;
        Ss[2 * tid] = r < Nq ? st[2 * r] : kInf;
        Ss[2 * tid + 1] = r < Nq ? st[2 * r + 1] : 0.f;
      }
      __syncthreads();
      for (int ii = 0; ii < kTile; ++ii) {
        const float* qr = Qs + ii * D + part * DT;
        const float* gr = Gs + ii * D + part * DT;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          s = __builtin_fmaf(kk[d], qr[d], s);
          dp = __builtin_fmaf(vv[d], gr[d], dp);
        }
        s = row_sum<TP>(s);
        dp = row_sum<TP>(dp);
        const bool vis = !CAUSAL || key <= r0 + ii + off;
        const float p = vis ? exp2_hw(__builtin_fmaf(s, a.c, -Ss[2 * ii])) : 0.f;
        const float ds = p * (dp - Ss[2 * ii + 1]);
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          dv[d] = __builtin_fmaf(p, gr[d], dv[d]);
          dk[d] = __builtin_fmaf(ds, qr[d], dk[d]);
        }
      }
      __syncthreads();
    }
  }
  if (real) {
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const int64_t e = kbase + (int64_t)key * D + part * DT + d;
      a.dk[e] = dk[d] * a.scale;
      a.dv[e] = dv[d];
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_typed(const BwdProblem& p, float* stat) {
  constexpr int RPB = F32Split<D>::RPB;
  BwdF32Args a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<const float*>(p.o);
  a.dout = static_cast<const float*>(p.dout);
  a.m = p.m;
  a.l = p.l;
  a.dq = static_cast<float*>(p.dq);
  a.dk = static_cast<float*>(p.dk);
  a.dv = static_cast<float*>(p.dv);
  a.stat = stat;
  a.H = (int)p.H;
  a.Hkv = (int)p.Hkv;
  a.group = (int)(p.H / p.Hkv);
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.nqt = (int)((p.Nq + RPB - 1) / RPB);
  a.nkt = (int)((p.Nk + RPB - 1) / RPB);
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  const int64_t g1 = p.B * p.H * a.nqt;
  if (g1 > 0) {
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, CAUSAL>), dim3((unsigned)g1), dim3(kThreads), 0,
                       p.stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t g2 = p.B * p.Hkv * a.nkt;
  if (g2 > 0) {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, CAUSAL>), dim3((unsigned)g2), dim3(kThreads), 0,
                       p.stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_d(const BwdProblem& p, float* stat) {
  return p.causal ? launch_typed<D, true>(p, stat) : launch_typed<D, false>(p, stat);
}

}  // namespace

hipError_t launch_bwd_f32(const BwdProblem& p, float* scratch) {
  switch (p.D) {
    case 16: return launch_d<16>(p, scratch);
    case 32: return launch_d<32>(p, scratch);
    case 64: return launch_d<64>(p, scratch);
    case 128: return launch_d<128>(p, scratch);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn

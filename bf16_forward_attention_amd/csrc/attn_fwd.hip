// attn_fwd.hip -- fused non-causal bf16 forward attention for MI355X (gfx950).
//
// O = softmax(Q K^T / sqrt(128)) V per (batch, head, query row), the
// operation the snilld.dk page "Open source attention kernel in HIP beats
// AITER v3 on MI300X" describes (section "Hvordan kernen arbejder" / How the
// kernel works), streamed over key tiles with a running maximum and sum so
// the score matrix never leaves registers (the FlashAttention family the same
// page places the design in, section "Memory-placement og mikroarkitektur").
//
// Work decomposition.  One workgroup of 4 wave64s owns BM = 128 query rows of
// one (batch, head); each wave owns 32 of them.  Keys stream in tiles of
// BN = 64 through LDS.  Both products run on v_mfma_f32_32x32x16_bf16 in the
// transposed orientation
//     S^T (keys x queries)  = K   . Q^T      A = K tile (LDS), B = Q (VGPRs)
//     O^T (dims x queries) += V^T . P^T      A = V^T tile (LDS), B = P (VGPRs)
// so that every lane owns exactly one query row: the softmax row statistics
// are per-lane scalars plus one exchange between the two 32-lane halves, and
// the rescale of the output accumulator is a per-lane multiply.
//
// MFMA 32x32x16 operand layout (lane l, g = l / 32):
//     A[i][k]: lane supplies row i = l % 32, k = 8g .. 8g+7
//     B[k][j]: lane supplies column j = l % 32, k = 8g .. 8g+7
//     C[i][j]: lane holds column j = l % 32, rows 8r + 4g + t in element 4r + t
//
// Key order inside a 32-key block.  The LDS K tile stores key
// pi(i) = 16*(i/4 % 2) + 4*(i/8) + i%4 in row i, so that after the first
// product lane group g holds the 16 consecutive keys 16g .. 16g+15 of the
// block in elements 0..15.  Eight of those consecutive keys are exactly a
// B operand for the second product, and the matching A operand is 8
// consecutive keys of one V^T row: one 16-byte LDS read.
//
// Numerics.  Logits accumulate in fp32 on the matrix cores.  The softmax runs
// in the base-2 domain: t = s * log2(e)/sqrt(128) (one fp32 constant), the
// running maximum m starts at -FLT_MAX (finite, so an all -Inf prefix never
// forms -Inf - -Inf) and is kept rounded up so the maximal key's weight is
// never above 1, p = exp2(t - m) on the hardware exp, the row sum l in
// fp32 from the unrounded p.  P is rounded to bf16 (nearest-even) for the
// second product.  The epilogue multiplies by 1/l and rounds once to bf16 in
// the requested mode.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "attn_fwd.h"

namespace {

constexpr int D = 128;
constexpr int BM = 128;                // query rows per workgroup
constexpr int BN = 64;                 // keys per tile
constexpr int NWAVES = BM / 32;        // 32 query rows per wave
constexpr int NTHREADS = NWAVES * 64;
constexpr int K_STRIDE = D + 8;        // bf16 per K row in LDS: 272 B, 4-bank skew per row
constexpr int VT_STRIDE = BN + 8;      // bf16 per V^T row in LDS: 144 B, 4-bank skew per row

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// log2(e) / sqrt(128), rounded to fp32
constexpr float kScaleLog2 = 0.12751743082459868f;

struct Geometry {
  int64_t q_row;   // element stride between consecutive query rows
  int64_t k_row;   // element stride between consecutive key rows
  int64_t q_head;  // element offset of head h within batch b: q_head * h
  int64_t k_head;
  int64_t q_batch; // element offset of batch b
  int64_t k_batch;
};

// Combine a per-lane value with the one held 32 lanes away (the other half of
// the wave).  This goes through ds_bpermute: AMD clang 22 folds
// fmaxf(r[0], r[1]) of __builtin_amdgcn_permlane32_swap(x, x) into r[0], as
// if the swap of a register with itself were the identity, which leaves the
// two halves with different values.
__device__ __forceinline__ float wave_half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
// fp32 addition is commutative, so both halves get identical bits
__device__ __forceinline__ float wave_half_sum(float x) { return x + __shfl_xor(x, 32); }

template <int MODE>
__device__ __forceinline__ uint16_t round_to_bf16(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (MODE == ATTN_ROUND_RTNE) {
    __bf16 b = (__bf16)x;  // v_cvt_pk_bf16_f32: nearest-even, NaN stays NaN
    return __builtin_bit_cast(uint16_t, b);
  }
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN: canonical quiet NaN
  if (MODE == ATTN_ROUND_RTNA) return (uint16_t)((u + 0x8000u) >> 16);
  return (uint16_t)(u >> 16);  // RTZ
}

// inverse of pi within a 32-key block: key a -> LDS row
__device__ __forceinline__ int k_row_of_key(int a) {
  return 8 * ((a & 15) >> 2) + 4 * (a >> 4) + (a & 3);
}

template <int MODE>
__global__ __launch_bounds__(NTHREADS, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, int H, int Sq, int Sk, int n_qtiles, Geometry g) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * K_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VT_STRIDE];

  // ---- workgroup -> (b, h, q-tile), keeping a head's q-tiles on one XCD ----
  // Workgroups are dispatched round-robin over the 8 XCDs; renumber so that
  // XCD x receives a contiguous range of logical work items.
  const int nwg = gridDim.x;
  const int id = blockIdx.x;
  const int xcd = id & 7, local = id >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  const int work = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int qt = work % n_qtiles;
  const int bh = work / n_qtiles;
  const int h = bh % H, b = bh / H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;

  const uint16_t* Qh = Q + b * g.q_batch + h * g.q_head;
  const uint16_t* Kh = K + b * g.k_batch + h * g.k_head;
  const uint16_t* Vh = V + b * g.k_batch + h * g.k_head;
  uint16_t* Oh = O + b * g.q_batch + h * g.q_head;

  // ---- Q fragments: this lane's query row, dims 16ks + 8grp .. +7 ----
  const int qrow = qt * BM + wave * 32 + l32;
  bf16x8 qf[8];
  {
    const bool ok = qrow < Sq;
    const uint16_t* src = Qh + (int64_t)(ok ? qrow : 0) * g.q_row + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 w = ok ? *(const u32x4*)(src + 16 * ks) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- tile staging assignment ----
  // K: thread covers 16-byte column chunk kc of keys kr0 + 16u (u = 0..3);
  //    16 consecutive threads read one 256-byte key row.
  const int kc = tid & 15, kr0 = tid >> 4;
  // V: thread covers column chunk vc (dims 8vc .. 8vc+7) of keys 4vg .. 4vg+3,
  //    transposed into V^T rows on the way into LDS.
  const int vg = tid & 15, vc = tid >> 4;

  u32x4 kbuf[4], vbuf[4];
  auto load_tile = [&](int base) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = base + kr0 + 16 * u;
      kbuf[u] = key < Sk ? *(const u32x4*)(Kh + (int64_t)key * g.k_row + 8 * kc) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = base + 4 * vg + u;
      vbuf[u] = key < Sk ? *(const u32x4*)(Vh + (int64_t)key * g.k_row + 8 * vc) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int a = kr0 + 16 * u;
      const int row = (a & 32) + k_row_of_key(a & 31);
      *(u32x4*)(k_lds + row * K_STRIDE + 8 * kc) = kbuf[u];
    }
    // vbuf[u][p] holds dims (8vc + 2p, 8vc + 2p + 1) of key 4vg + u
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t w0 = vbuf[0][p], w1 = vbuf[1][p], w2 = vbuf[2][p], w3 = vbuf[3][p];
      u32x2 even = {(w0 & 0xFFFFu) | (w1 << 16), (w2 & 0xFFFFu) | (w3 << 16)};
      u32x2 odd = {(w0 >> 16) | (w1 & 0xFFFF0000u), (w2 >> 16) | (w3 & 0xFFFF0000u)};
      *(u32x2*)(vt_lds + (8 * vc + 2 * p) * VT_STRIDE + 4 * vg) = even;
      *(u32x2*)(vt_lds + (8 * vc + 2 * p + 1) * VT_STRIDE + 4 * vg) = odd;
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  float m_run = -3.402823466e38f;
  float l_run = 0.0f;

  const int n_tiles = (Sk + BN - 1) / BN;
  load_tile(0);
  for (int t = 0; t < n_tiles; ++t) {
    const int base = t * BN;
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(base + BN);  // in flight while this tile computes

    // ---- S^T = K . Q^T for the two 32-key blocks ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const uint16_t* krow = k_lds + (32 * kb + l32) * K_STRIDE + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8 a = *(const bf16x8*)(krow + 16 * ks);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }

    // keys past Sk (only in the last tile) get a -Inf logit
    if (base + BN > Sk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int n = 0; n < 16; ++n)
          if (base + 32 * kb + 16 * grp + n >= Sk) s[kb][n] = -__builtin_inff();
    }

    // ---- online softmax (base 2) ----
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int n = 0; n < 16; ++n) mx = fmaxf(mx, s[kb][n]);
    mx = wave_half_max(mx);
    // The new maximum is the scaled row maximum rounded up by at least half
    // an ulp: then fma(s, c, -m) <= 0 for the maximal logit, its weight is
    // exp2(<= 0) <= 1 and rounds to exactly 1 in bf16, so a row dominated by
    // one key (or with a single key) returns that V row exactly in every mode.
    // (-Inf / NaN maxima give NaN here, which fmaxf ignores.)
    const float mx_scaled = mx * kScaleLog2;
    const float m_new = fmaxf(m_run, __builtin_fmaf(__builtin_fabsf(mx_scaled), 0x1p-23f, mx_scaled));
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    float psum = 0.0f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const int n = 8 * hh + 2 * q2;
          f32x2 p;
          p[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][n], kScaleLog2, -m_new));
          p[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][n + 1], kScaleLog2, -m_new));
          psum += p[0];
          psum += p[1];
          bf16x2 pb = __builtin_convertvector(p, bf16x2);
          pf[kb][hh][2 * q2] = pb[0];
          pf[kb][hh][2 * q2 + 1] = pb[1];
        }
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] *= alpha;

    // ---- O^T += V^T . P^T ----
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint16_t* vrow = vt_lds + (32 * db + l32) * VT_STRIDE + 16 * grp;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 a = *(const bf16x8*)(vrow + 32 * kb + 8 * hh);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][hh], acc[db], 0, 0, 0);
        }
    }
  }

  // ---- epilogue: normalise, round, store this lane's query row ----
  const float l_tot = wave_half_sum(l_run);
  const float inv_l = 1.0f / l_tot;
  if (qrow < Sq) {
    uint16_t* dst = Oh + (int64_t)qrow * g.q_row + 4 * grp;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t lo = round_to_bf16<MODE>(acc[db][4 * r + 0] * inv_l) |
                      ((uint32_t)round_to_bf16<MODE>(acc[db][4 * r + 1] * inv_l) << 16);
        uint32_t hi = round_to_bf16<MODE>(acc[db][4 * r + 2] * inv_l) |
                      ((uint32_t)round_to_bf16<MODE>(acc[db][4 * r + 3] * inv_l) << 16);
        *(u32x2*)(dst + 32 * db + 8 * r) = u32x2{lo, hi};
      }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev < kMaxDevices) {
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 1) return ATTN_OK;
    if (st == 2) return ATTN_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_release);
  return ok ? ATTN_OK : ATTN_ERR_DEVICE;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

}  // namespace

extern "C" int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                             int64_t Sq, int64_t Sk, int layout, int round_mode, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ATTN_ERR_SIZE;
  int64_t bh, nq, nk, bytes_q, bytes_k;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, Sq, &nq) || !mul_ok(nq, 2 * D, &bytes_q) || !mul_ok(bh, Sk, &nk) ||
      !mul_ok(nk, 2 * D, &bytes_k))
    return ATTN_ERR_SIZE;
  const int64_t n_qtiles = (Sq + BM - 1) / BM;
  int64_t n_wg;
  if (!mul_ok(bh, n_qtiles, &n_wg) || n_wg > INT32_MAX || Sq > INT32_MAX || Sk > INT32_MAX || H > INT32_MAX)
    return ATTN_ERR_SIZE;
  if (layout != ATTN_LAYOUT_BSHD && layout != ATTN_LAYOUT_BHSD) return ATTN_ERR_LAYOUT;
  if (round_mode != ATTN_ROUND_RTNE && round_mode != ATTN_ROUND_RTNA && round_mode != ATTN_ROUND_RTZ)
    return ATTN_ERR_ROUND;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return ATTN_ERR_ALIGN;
  if (overlaps(o, bytes_q, q, bytes_q) || overlaps(o, bytes_q, k, bytes_k) || overlaps(o, bytes_q, v, bytes_k))
    return ATTN_ERR_ALIAS;
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;

  Geometry g;
  if (layout == ATTN_LAYOUT_BSHD) {
    g.q_row = H * D;
    g.k_row = H * D;
    g.q_head = D;
    g.k_head = D;
    g.q_batch = Sq * H * D;
    g.k_batch = Sk * H * D;
  } else {
    g.q_row = D;
    g.k_row = D;
    g.q_head = Sq * D;
    g.k_head = Sk * D;
    g.q_batch = H * Sq * D;
    g.k_batch = H * Sk * D;
  }
  const dim3 grid((unsigned)n_wg), block(NTHREADS);
  hipStream_t s = (hipStream_t)stream;
  const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k, *vv = (const uint16_t*)v;
  uint16_t* oo = (uint16_t*)o;
  switch (round_mode) {
    case ATTN_ROUND_RTNE:
      hipLaunchKernelGGL(attn_fwd_kernel<ATTN_ROUND_RTNE>, grid, block, 0, s, qq, kk, vv, oo, (int)H, (int)Sq,
                         (int)Sk, (int)n_qtiles, g);
      break;
    case ATTN_ROUND_RTNA:
      hipLaunchKernelGGL(attn_fwd_kernel<ATTN_ROUND_RTNA>, grid, block, 0, s, qq, kk, vv, oo, (int)H, (int)Sq,
                         (int)Sk, (int)n_qtiles, g);
      break;
    default:
      hipLaunchKernelGGL(attn_fwd_kernel<ATTN_ROUND_RTZ>, grid, block, 0, s, qq, kk, vv, oo, (int)H, (int)Sq,
                         (int)Sk, (int)n_qtiles, g);
      break;
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" const char* attn_fwd_bf16_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a tensor pointer is NULL";
    case ATTN_ERR_SIZE: return "B, H, Sq and Sk must be >= 1 and the problem must fit the index types";
    case ATTN_ERR_LAYOUT: return "layout must be ATTN_LAYOUT_BSHD or ATTN_LAYOUT_BHSD";
    case ATTN_ERR_ROUND: return "round_mode must be ATTN_ROUND_RTNE, ATTN_ROUND_RTNA or ATTN_ROUND_RTZ";
    case ATTN_ERR_ALIGN: return "q, k, v and o must be 16-byte aligned";
    case ATTN_ERR_ALIAS: return "o overlaps q, k or v";
    case ATTN_ERR_DEVICE: return "the current HIP device is not gfx950 (MI355X) or cannot be queried";
    case ATTN_ERR_HIP: return "the HIP kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int attn_fwd_bf16_abi_version(void) { return ATTN_FWD_ABI_VERSION; }

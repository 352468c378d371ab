// Grouped output projection: Y[:, gi*d_g:(gi+1)*d_g] = X_gi . W_gi^T for the g head groups.
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.3 (the c*n_h
// concatenated head outputs are split into g groups of heads, each projected by its own
// smaller d_g x (c*n_h/g) matrix, the g results concatenated) and section IV (the
// projection is shared by both branches).
//
// Two kernels, both on v_mfma_f32_16x16x32_bf16:
//   * gop_skinny (few tokens: decode): bound by streaming W once.  A workgroup owns 16
//     output columns of one group for every token; its four waves split K and meet in
//     LDS.  Each lane streams 16 B of one weight row per step, eight steps in flight.
//   * gop_gemm (many tokens: prefill): bound by MFMA.  A workgroup computes a 256 x 256
//     tile (tokens x columns) as 2 x 4 waves of 128 x 64 (two waves per SIMD, so one's LDS
//     reads overlap the other's MFMAs), over K in stages of 64 that global_load_lds moves
//     straight into LDS, double-buffered.  A stage reads each row's slice as one 128-byte
//     line (stages of 32 with twice the requests measured 20% slower).  LDS rows are 128 B
//     with their 16-byte chunks XOR-swizzled by (row / 2) mod 8, so that the 16 rows a
//     fragment read touches fall in 16 distinct bank groups.  Tiles are handed out so that each XCD
//     gets a contiguous run; the column tiles of a token tile run together there and share
//     its rows in that XCD's L2.
#include <mutex>

#include "common.hpp"

namespace {

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------------------
// skinny: T tokens in M tiles of 16, up to MT tiles per workgroup
// ---------------------------------------------------------------------------------------
constexpr int SK_U = 8;  // K steps (of 32) in flight per wave

template <int MT>
__global__ __launch_bounds__(256) void gop_skinny(const uint16_t* __restrict__ X,
                                                  const uint16_t* __restrict__ Wt,
                                                  uint16_t* __restrict__ Y, int T, int K_g,
                                                  int d_g, long long ldx, long long ldy,
                                                  int ctiles) {
  __shared__ f32x4 red[4][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int gi = blockIdx.x / ctiles, ct = blockIdx.x - gi * ctiles;
  const int t0 = blockIdx.y * (16 * MT);
  const int Kq = K_g / 4;  // this wave's quarter of K
  const int kbeg = wave * Kq;
  const uint16_t* wrow = Wt + ((size_t)gi * d_g + ct * 16 + r16) * K_g + kbeg + kg * 8;
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int t = t0 + mt * 16 + r16;
    xok[mt] = t < T;
    xrow[mt] = X + (size_t)(xok[mt] ? t : 0) * ldx + (size_t)gi * K_g + kbeg + kg * 8;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = MT <= 2 ? SK_U : SK_U / 2;
  int k = 0;
  for (; k + 32 * U <= Kq; k += 32 * U) {
    u32x4 b[U], a[MT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = *reinterpret_cast<const u32x4*>(wrow + k + u * 32);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int u = 0; u < U; ++u)
        a[mt][u] = xok[mt] ? *reinterpret_cast<const u32x4*>(xrow[mt] + k + u * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mt][u]),
                                                          __builtin_bit_cast(bf16x8, b[u]), acc[mt], 0, 0, 0);
  }
  for (; k < Kq; k += 32) {  // the quarter's last steps
    const u32x4 b = *reinterpret_cast<const u32x4*>(wrow + k);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 a = xok[mt] ? *reinterpret_cast<const u32x4*>(xrow[mt] + k) : u32x4{0, 0, 0, 0};
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), acc[mt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[wave][mt][lane] = acc[mt];
  __syncthreads();
  // wave w sums the four K quarters of M tile w (and w + 4, ...); fixed order
  for (int mt = wave; mt < MT; mt += 4) {
    f32x4 s = red[0][mt][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 o = red[w][mt][lane];
      s = f32x4{s[0] + o[0], s[1] + o[1], s[2] + o[2], s[3] + o[3]};
    }
    // accumulator layout: column r16, rows 4 * kg + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + mt * 16 + 4 * kg + i;
      if (t < T) Y[(size_t)t * ldy + (size_t)gi * d_g + ct * 16 + r16] = f32_to_bf16(s[i]);
    }
  }
}

// ---------------------------------------------------------------------------------------
// gemm: 256 x 256 tiles, 8 waves of 128 x 64, K stages of 64 double-buffered in LDS
// ---------------------------------------------------------------------------------------
constexpr int GM = 256, GN = 256, GK = 64, GNS = 2, GWAVES = 8;
constexpr int ROWB = GK * 2;                               // 128 B per staged row
constexpr int A_BYTES = GM * ROWB, B_BYTES = GN * ROWB;   // 32 KiB + 32 KiB
constexpr int STAGE = A_BYTES + B_BYTES;
constexpr int GEMM_LDS = GNS * STAGE;                      // 128 KiB
constexpr int LPR = ROWB / 16, RPI = 64 / LPR;            // lanes per row, rows per DMA
constexpr int A_DMA = A_BYTES / 1024 / GWAVES, B_DMA = B_BYTES / 1024 / GWAVES;  // 4, 4

// position of 16-byte chunk kc (0..7) in staged row r: the 16 rows a fragment read
// touches (2 per 256 bytes) land on 16 distinct 16-byte bank groups
CSAHCA_DEV int swz(int r, int kc) { return kc ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(512, 1) void gop_gemm(const uint16_t* __restrict__ X,
                                                   const uint16_t* __restrict__ Wt,
                                                   uint16_t* __restrict__ Y, int T, int K_g,
                                                   int d_g, long long ldx, long long ldy,
                                                   int mtiles, int ntiles, int tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  // XCD-contiguous tile order (the hardware deals workgroups round-robin over 8 XCDs)
  int tile = blockIdx.x;
  if (tiles % 8 == 0) tile = (blockIdx.x & 7) * (tiles >> 3) + (blockIdx.x >> 3);
  const int nt = tile % ntiles;
  const int mt = (tile / ntiles) % mtiles;
  const int gi = tile / (ntiles * mtiles);
  const int m0 = mt * GM, n0 = nt * GN;

  // DMA: instruction q (of a stage's 32 A and 32 B ones) moves rows RPI*q .. RPI*q+7; lane
  // L row RPI*q + L/LPR, LDS position L%LPR holding data chunk swz(row, L%LPR).  Each row
  // slice is one 128-byte line.
  const uint16_t* asrc[A_DMA];
  const uint16_t* bsrc[B_DMA];
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) {
    const int r = RPI * (wave * A_DMA + i) + lane / LPR;
    const int t = min(m0 + r, T - 1);  // rows past the end repeat the last (results dropped)
    asrc[i] = X + (size_t)t * ldx + (size_t)gi * K_g + swz(r, lane % LPR) * 8;
  }
#pragma unroll
  for (int i = 0; i < B_DMA; ++i) {
    const int r = RPI * (wave * B_DMA + i) + lane / LPR;
    bsrc[i] = Wt + ((size_t)gi * d_g + n0 + r) * K_g + swz(r, lane % LPR) * 8;
  }
  auto issue = [&](int s) {
    uint8_t* st = smem + (s % GNS) * STAGE;
    const int k0 = s * GK;
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
      __builtin_amdgcn_global_load_lds(asrc[i] + k0, (lds_void*)(st + (wave * A_DMA + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i)
      __builtin_amdgcn_global_load_lds(bsrc[i] + k0, (lds_void*)(st + A_BYTES + (wave * B_DMA + i) * 1024), 16,
                                       0, 0);
  };

  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves of 128 x 64
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nst = K_g / GK;
  issue(0);
  for (int s = 0; s < nst; ++s) {
    // stage s landed for every wave; then stage s + 1 streams in while s is computed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (s + 1 < nst) issue(s + 1);  // into the buffer every wave left at s - 1
    const uint8_t* st = smem + (s % GNS) * STAGE;
#pragma unroll
    for (int ks = 0; ks < GK / 32; ++ks) {
      const int kc = ks * 4 + kg;
      u32x4 a[8], b[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wm * 128 + i * 16 + r16;
        a[i] = *reinterpret_cast<const u32x4*>(st + r * ROWB + swz(r, kc) * 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + r16;
        b[j] = *reinterpret_cast<const u32x4*>(st + A_BYTES + r * ROWB + swz(r, kc) * 16);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                              __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
    }
  }
  // accumulator layout: column r16, rows 4 * kg + e of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = m0 + wm * 128 + i * 16 + 4 * kg + e;
      if (t < T) {
        uint16_t* yr = Y + (size_t)t * ldy + (size_t)gi * d_g + n0 + wn * 64 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) yr[j * 16] = f32_to_bf16(acc[i][j][e]);
      }
    }
}


}  // namespace

extern "C" int grouped_out_proj(const void* o, const void* w, void* y, int T, int g, int K_g,
                                int d_g, long long ldo, long long ldy, int dtype, void* stream) {
  using namespace csahca;
  const char* name = "grouped_out_proj";
  if (T < 0 || g < 1 || K_g < 1 || d_g < 1) return fail(CSAHCA_EINVAL, "grouped_out_proj: need T >= 0 and g, K_g, d_g >= 1");
  if (dtype != CSAHCA_BF16) return fail(CSAHCA_ENOTSUP, "grouped_out_proj: dtype must be CSAHCA_BF16");
  if (K_g % 128 != 0 || d_g % 16 != 0)
    return fail(CSAHCA_ENOTSUP, "grouped_out_proj: needs K_g % 128 == 0 and d_g % 16 == 0");
  if (ldo < (long long)g * K_g || ldy < (long long)g * d_g || ldo % 8 || ldy % 8)
    return fail(CSAHCA_EINVAL, "grouped_out_proj: ldo >= g*K_g and ldy >= g*d_g, multiples of 8");
  if (T == 0) {
    clear_error();
    return CSAHCA_OK;
  }
  if (!o || !w || !y) return fail(CSAHCA_EINVAL, "grouped_out_proj: o, w and y must be non-NULL");
  if (!aligned16(o) || !aligned16(w) || !aligned16(y))
    return fail(CSAHCA_EINVAL, "grouped_out_proj: o, w and y must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const uint16_t *X = (const uint16_t*)o, *Wt = (const uint16_t*)w;
  uint16_t* Y = (uint16_t*)y;
  if (T > 64 && d_g % GN == 0 && K_g % GK == 0) {
    const long long mtiles = cdiv<long long>(T, GM), ntiles = d_g / GN, tiles = mtiles * ntiles * g;
    if (tiles > 0x7FFFFFFFLL) return fail(CSAHCA_ENOTSUP, "grouped_out_proj: problem too large");
    // raise the kernel's dynamic LDS limit once per process, whichever thread calls first
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
      attr = hipFuncSetAttribute((const void*)gop_gemm, hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS);
    });
    if (attr != hipSuccess) return fail(CSAHCA_ELAUNCH, "grouped_out_proj: cannot set the LDS size");
    hipLaunchKernelGGL(gop_gemm, dim3((unsigned)tiles), dim3(64 * GWAVES), GEMM_LDS, st, X, Wt, Y, T, K_g, d_g, ldo, ldy,
                       (int)mtiles, (int)ntiles, (int)tiles);
    return launch_status(name);
  }
  const int ctiles = d_g / 16;
  const long long groups = cdiv<long long>(T, 64);
  if ((long long)g * ctiles > 0x7FFFFFFFLL || groups > 65535)
    return fail(CSAHCA_ENOTSUP, "grouped_out_proj: problem too large for the few-token kernel");
  const int tl = T - (int)(groups - 1) * 64;  // tokens of the last 64-token group
  const int MT = (int)groups > 1 ? 4 : (tl + 15) / 16;
  const dim3 grid((unsigned)(g * ctiles), (unsigned)groups);
  switch (MT) {
    case 1:
      hipLaunchKernelGGL(gop_skinny<1>, grid, dim3(256), 0, st, X, Wt, Y, T, K_g, d_g, ldo, ldy, ctiles);
      break;
    case 2:
      hipLaunchKernelGGL(gop_skinny<2>, grid, dim3(256), 0, st, X, Wt, Y, T, K_g, d_g, ldo, ldy, ctiles);
      break;
    case 3:
      hipLaunchKernelGGL(gop_skinny<3>, grid, dim3(256), 0, st, X, Wt, Y, T, K_g, d_g, ldo, ldy, ctiles);
      break;
    default:
      hipLaunchKernelGGL(gop_skinny<4>, grid, dim3(256), 0, st, X, Wt, Y, T, K_g, d_g, ldo, ldy, ctiles);
  }
  return launch_status(name);
}

// Fast bf16 WBMM forward for w = 14, NCHW, square images of 28x28 or 56x56, table input, bf16
// output, no 3x3 mix. With bf16 operands the window contraction needs little matrix time
// (v_mfma_f32_16x16x32_bf16 does 16x16x32 per instruction); what bounds such a kernel is moving
// the map through HBM and the LDS instruction pipe (about 7-8 cycles per CU for one LDS
// instruction of any width up to 16 bytes per lane). So only the table lives in LDS:
//   * a unit = 64 windows of one channel (4 wave-units of 16 windows, whole images); persistent
//     workgroups each walk a run of consecutive units (one channel, so the table is staged once),
//     every wave keeping the next unit's pixels in flight while it contracts the current one;
//   * the window operand of the MFMA goes from HBM straight into registers: lane (window n, K
//     group g) needs 8 pixels of one window row per K step (rows padded to 16 pixels, K = 224 =
//     7 steps of 32), which is one 16-byte load at pixel 0 of the row half or, for the second
//     half, at pixel 6 followed by a one-dword shift that also zeroes the two padding slots (the
//     load never leaves the window row);
//   * M_c is never formed: the table is reversed with its rows padded to a pitch of 32, and 8
//     copies shifted by 0..7 make any 8-entry run of a row one aligned 16-byte LDS read
//     [gecl.asia reading notes, "Core Idea"; the notes' "Limitation" and "Takeaway" name such a
//     kernel as future work]. With pitch 32 a pixel needs the same copy in every window row and
//     K step, so all of a lane's table reads are one base plus immediates;
//   * output tiles are window rows: MFMA rows 0..11 are pixels 0..11 of the row and rows 12..15
//     pixels 10..13 again, so a lane's four accumulators are 4 consecutive pixels of one window
//     row, rounded to bf16 (RNE, v_cvt_pk_bf16_f32); tiles leave in pairs, the odd lane groups
//     of one tile swapped with the even groups of the next (v_permlane16_swap), so each lane
//     stores 8 consecutive pixels of one row as one 16-byte store straight to HBM (pixels 10, 11
//     are written twice with the same value). Images past the batch read and write the batch's
//     last image (same values again), so no store needs a branch and the wait for the next
//     unit's loads never waits for stores.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

#include <type_traits>
#include <utility>

namespace wbmm {
namespace {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
// 16- and 8-byte accesses at 4-byte alignment (window rows start at even 28-byte offsets)
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));
// 8-byte stores at 2-byte alignment (w = 7 window rows start at 14-byte offsets); the HSA
// runtime runs global memory in unaligned-access mode
typedef uint32_t u32x2a2 __attribute__((ext_vector_type(2), aligned(2)));

struct BfArgs {
  int B, C;
  int groups;  // units per channel: ceil(B / images per unit)
  const uint16_t* x;
  const uint16_t* T;
  uint16_t* y;
  uint16_t* z;  // optional copy of the output (the pre-mix map equals y without a mix)
  const float* mixw;  // (C, 3, 3) weights of the fused 3x3 mix (MIX kernels), else null
};

template <int IW_>
struct BfShape {
  static constexpr int WS = 14, IH = IW_, IW = IW_;
  static constexpr int L1 = 2 * WS - 1;
  static constexpr int NWX = IW / WS, NWIN = NWX * NWX;
  static constexpr int IPW = 16 / NWIN;           // images per wave-unit
  static constexpr int PLANE = IH * IW;
  static constexpr int TP = 32;                   // padded table row pitch
  static constexpr int PT = L1 * TP;              // padded table entries
  static constexpr int CS = 952;                  // bf16 per shifted copy (copy r starts r*CS)
  // reversed padded table: M[i][(yj, xj)] = Rv[bi + TP yj + xj] with bi = C0 - TP yi - xi and
  // Rv[q] = Tpad[PT-1-q]
  static constexpr int C0 = PT - 1 - (WS - 1) * TP - (WS - 1);
  static_assert(IW == 28 || IW == 56, "shape");
  static_assert(CS % 8 == 0 && CS >= PT + 16, "copies");
  // fused 3x3 mix: each wave stages the pre-mix map of its images as bf16 planes with a zero
  // halo, image column v at plane column v + 2 (so 2-pixel runs are 4-byte aligned), pitch ZP
  static constexpr int ZP = IW + 4, ZPLANE = (IH + 2) * ZP;
  static constexpr int ZWAVE = IPW * ZPLANE;      // bf16 per wave
  static constexpr int CPAIR = IW / 2;            // column pairs per image row
  static constexpr int RSEG = 64 / (IPW * CPAIR); // row segments per column pair (1 or 2)
  static constexpr int RLEN = IH / RSEG;
  static_assert(RSEG >= 1 && IH % RSEG == 0 && IPW * CPAIR * RSEG <= 64, "mix tasks");
};

template <class S>
constexpr int bf_lds_bytes() { return 8 * S::CS * 2; }
// with the fused mix: the table copies, then 4 waves' staging planes
template <class S>
constexpr int bf_mix_lds_bytes() { return 8 * S::CS * 2 + 4 * S::ZWAVE * 2; }

// Pixel offset of window n's first pixel within its image plane (window n of a wave-unit lies in
// image n / NWIN of it).
template <class S>
__device__ __forceinline__ int win_off(int n) {
  const int k = n % S::NWIN;
  return (k / S::NWX) * S::WS * S::IW + (k % S::NWX) * S::WS;
}

// Where unit u's data live: channel c, first image, images in the unit.
struct UnitPos {
  int c, img0, nimg;
};
__device__ __forceinline__ UnitPos unit_pos(const BfArgs& a, int u, int ipu) {
  UnitPos p;
  p.c = u / a.groups;
  p.img0 = (u - p.c * a.groups) * ipu;
  p.nimg = min(a.B - p.img0, ipu);
  return p;
}

// A value hidden from the optimizer at this point of the program (it cannot be computed
// earlier than here).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Stages channel c's table into LDS as 8 copies of the reversed table with rows padded to pitch
// TP, copy r shifted by r entries: copy r holds Rv[q] = Tpad[PT-1-q] at q + r, so an 8-entry run
// of Rv that starts at q is one aligned 16-byte read from copy (-q) & 7. Entries q >= CS - 7 lie
// past every read; threads past CS - 8 repeat entry CS - 8 (same value to the same places), so
// every write is unconditional. All threads of the workgroup take part. Split in two so that a
// caller can put other loads in flight between them: the memory counter completes in order, so
// waiting for the table entries never waits for loads issued after them. ROT stages the table
// rotated by 180 degrees (entry L-1-q for q), whose matrix is M^T: the contraction then computes
// the backward's dX = M^T G.
template <class S, int NTH, bool ROT = false>
struct TableStage {
  static constexpr int NQ = (S::CS + NTH - 1) / NTH;
  uint16_t tv[NQ];
  uint32_t pad;  // bit j: entry j is padding (zero); applied at write time, so that nothing
                 // waits for the loads before write
  __device__ __forceinline__ void load(const uint16_t* T, int c) {
    const uint16_t* Tc = T + (size_t)c * S::L1 * S::L1;
    // the thread index is made opaque so that the per-entry indices are computed here, not kept
    // in registers from the kernel's start (a persistent caller stages rarely)
    const int tid = opaque(threadIdx.x);
    pad = 0;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = min(tid + j * NTH, S::CS - 8);
      const int p = S::PT - 1 - q;  // padded table index
      const bool in = p >= 0 && (p % S::TP) < S::L1;
      const int ti = in ? (p / S::TP) * S::L1 + (p % S::TP) : 0;
      tv[j] = Tc[ROT ? S::L1 * S::L1 - 1 - ti : ti];
      pad |= in ? 0u : 1u << j;
    }
  }
  __device__ __forceinline__ void write(uint16_t* copies) const {
    __syncthreads();  // every wave is done with the previous copies
    const int tid = opaque(threadIdx.x);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = min(tid + j * NTH, S::CS - 8);
      const uint16_t v = (pad >> j) & 1u ? (uint16_t)0 : tv[j];
#pragma unroll
      for (int r = 0; r < 8; ++r) copies[r * S::CS + q + r] = v;
    }
    __syncthreads();
  }
};
template <class S, int NTH = kThreads, bool ROT = false>
__device__ __forceinline__ void stage_table(uint16_t* copies, const uint16_t* T, int c) {
  TableStage<S, NTH, ROT> ts;
  ts.load(T, c);
  ts.write(copies);
}

// Persistent: workgroup g walks the units [g*units/grid, (g+1)*units/grid) (a run of consecutive
// units shares a channel, so the table copies are rebuilt only when it changes); each wave owns
// one wave-unit (16 windows) of every unit and has the next unit's pixels in flight while it
// contracts and stores the current one.
constexpr int kWgPerCu = 4;  // resident workgroups per CU (kWgPerCu waves per SIMD)
constexpr int kWgPerCuMix = 3;  // with the fused mix's staging planes

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// MIX: the 3x3 inter-block mix is fused [gecl.asia reading notes, "Method" point 3]: the output
// tiles (z, rounded to bf16) go to the wave's staging planes instead of memory (z_save still
// gets them), and once the wave has contracted its images it computes
// y[h][v] = sum_{u,t} W[u][t] z[h+u-1][v+t-1] (fp32 sums of the bf16 z, zero outside the image,
// RNE to bf16) from the planes: a lane walks a pair of columns down its image with a sliding
// 3 x 4 register window (three 4-byte LDS reads per row) and stores the pair as 4 bytes.
template <class S, bool ZS, bool ROT = false, bool MIX = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MIX ? kWgPerCuMix : kWgPerCu, 8)))
k_fwd_bf16(BfArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_h[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  uint16_t* copies = smem_h;  // [8][CS]
  const int units = a.C * a.groups;
  const int u0 = (int)((long long)blockIdx.x * units / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * units / gridDim.x);
  if (u0 >= u1) return;  // uniform over the workgroup
  constexpr int IPU = 4 * S::IPW;  // images per unit

  // lane (n, gq): MFMA column n = window n of the wave-unit, MFMA row n = pixel slot n of the
  // tile's window row; lane group gq = K block 4s + gq of step s = window row 2s + kq, pixels
  // 8kh .. 8kh + 7, and output slots 4gq .. 4gq + 3 = pixels px0 .. px0 + 3
  const int n = lane & 15, gq = lane >> 4;
  const int kq = gq >> 1, kh = gq & 1;
  const int im = wave * S::IPW + n / S::NWIN;  // image of window n within the unit
  const int xo = win_off<S>(n) + kq * S::IW + 6 * kh;
  // tiles leave in pairs (t, t + 1): lane group gq stores 8 pixels of tile t + (gq & 1),
  // pixels 0..7 (gq < 2) or 6..13
  const int so = win_off<S>(n) + (gq & 1) * S::IW + (gq < 2 ? 0 : S::WS - 8);
  // table run of tile t (pixel (t, xi)), step s at ab + TP (WS-1-t) + 2 TP s; immediates >= 0
  const int xi = n < 8 ? n : n - 2;
  const int bi0 = S::C0 - xi;          // row t subtracts TP t, which keeps the copy index
  const int rc = (-bi0) & 7;           // copy whose runs from bi (mod 8) are 16-byte aligned
  const int ab = rc * S::CS + bi0 + rc + S::TP * kq + 8 * kh - S::TP * (S::WS - 1);

  // MIX: this wave's staging planes, zeroed once (the halo stays zero: tiles only write the
  // interior); zoff: where this lane's 8 output pixels of tile 0 go
  uint16_t* zst = copies + 8 * S::CS + wave * S::ZWAVE;
  int zoff = 0;
  if constexpr (MIX) {
    for (int e = lane; e < S::ZWAVE / 2; e += 64) ((uint32_t*)zst)[e] = 0u;
    const int k = n % S::NWIN;
    const int row0 = (k / S::NWX) * S::WS + (gq & 1);
    const int col0 = (k % S::NWX) * S::WS + (gq < 2 ? 0 : S::WS - 8);
    zoff = (n / S::NWIN) * S::ZPLANE + (row0 + 1) * S::ZP + col0 + 2;
    wave_lds_sync();
  }

  auto plane = [&](const UnitPos& p) {  // element offset of this lane's image plane
    const int ic = min(im, p.nimg - 1);  // images past the batch read its last image
    return ((size_t)(p.img0 + ic) * a.C + p.c) * S::PLANE;
  };
  auto issue = [&](const UnitPos& p, u32x4 (&raw)[7]) {
    const uint16_t* src = a.x + plane(p) + xo;
#pragma unroll
    for (int s = 0; s < 7; ++s) raw[s] = *(const u32x4a*)(src + 2 * s * S::IW);
  };
  // window operand: pixels 8kh .. 8kh+7 of the row; the second half was loaded from pixel 6
  u32x4 xv[7];
  auto convert = [&](const u32x4 (&raw)[7]) {
#pragma unroll
    for (int s = 0; s < 7; ++s) {
      xv[s].x = kh ? raw[s].y : raw[s].x;
      xv[s].y = kh ? raw[s].z : raw[s].y;
      xv[s].z = kh ? raw[s].w : raw[s].z;
      xv[s].w = kh ? 0u : raw[s].w;
    }
  };

  int table_c = -1;
  // One unit: stage its channel's table if needed, put unit u_next's pixels in flight into
  // `into` (when `more`), contract and store, then convert `conv` (the pixels of the next unit
  // to contract) into the operand. The conversion comes after this unit's stores are issued, so
  // its wait counts only loads; the last unit of a run is peeled off so that no load is ever
  // conditional (a conditional load makes the wait counting fall back to waiting for all).
  auto unit = [&](auto more, const UnitPos& pos, int u_next, u32x4 (&into)[7],
                  const u32x4 (&conv)[7]) {
    if (pos.c != table_c) {  // uniform over the workgroup
      stage_table<S, kThreads, ROT>(copies, a.T, pos.c);
      table_c = pos.c;
    }
    constexpr bool MORE = decltype(more)::value;
    const UnitPos nxt = unit_pos(a, u_next < u1 ? u_next : u1 - 1, IPU);
    if constexpr (MORE) issue(nxt, into);

    const size_t obase = plane(pos) + so;
    // out[window n][pixel (t, 4gq + r)] = sum_k M[(t, 4gq + r)][k] X[k][window n]
    auto half = [&](auto t0c, auto ntc) {
      constexpr int T0 = decltype(t0c)::value, NT = decltype(ntc)::value;
      // (s, t) steps, t fastest; table reads PD steps ahead
      constexpr int N = 7 * NT, PD = S::IW == 56 ? 3 : 2;
      v4f acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
      u32x4 mv[PD + 1];
#pragma unroll
      for (int k = 0; k < PD; ++k)
        mv[k] = *(const u32x4*)(copies + ab + S::TP * (S::WS - 1 - T0 - k % NT) + 2 * S::TP * (k / NT));
#pragma unroll
      for (int k = 0; k < N; ++k) {
        if (k + PD < N) {
          const int kn = k + PD;
          mv[kn % (PD + 1)] =
              *(const u32x4*)(copies + ab + S::TP * (S::WS - 1 - T0 - kn % NT) + 2 * S::TP * (kn / NT));
        }
        acc[k % NT] = mfma_bf16(mv[k % (PD + 1)], xv[k / NT], acc[k % NT]);
        // keep this order: the scheduler otherwise trades the read-ahead for registers
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane group gq holds pixels 4gq .. 4gq+3 (groups 2, 3: 6 .. 13) of tile t; swapping the
      // odd groups of tile t with the even groups of tile t + 1 (v_permlane16_swap) leaves every
      // lane 8 consecutive pixels of one tile: one 16-byte store per lane and tile pair
      static_assert(NT % 2 == 0, "tile pairs");
#pragma unroll
      for (int t = 0; t < NT; t += 2) {
        uint32_t pk[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          pk[u][0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{acc[t + u][0], acc[t + u][1]}), v2bf));
          pk[u][1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{acc[t + u][2], acc[t + u][3]}), v2bf));
        }
        const auto lo = __builtin_amdgcn_permlane16_swap(pk[0][0], pk[1][0], false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(pk[0][1], pk[1][1], false, false);
        const u32x4 v = u32x4{lo[0], hi[0], lo[1], hi[1]};
        const size_t o = obase + (size_t)(T0 + t) * S::IW;
        if constexpr (MIX) {
          uint32_t* zp = (uint32_t*)(zst + zoff + (T0 + t) * S::ZP);
          zp[0] = v.x;
          zp[1] = v.y;
          zp[2] = v.z;
          zp[3] = v.w;
        } else {
          *(u32x4a*)(a.y + o) = v;
        }
        if constexpr (ZS) *(u32x4a*)(a.z + o) = v;
      }
    };
    half(std::integral_constant<int, 0>{}, std::integral_constant<int, 8>{});
    half(std::integral_constant<int, 8>{}, std::integral_constant<int, 6>{});
    if constexpr (MIX) {
      wave_lds_sync();  // every lane's tiles are in the planes
      if (lane < S::IPW * S::CPAIR * S::RSEG) {
        const int i = lane / (S::CPAIR * S::RSEG), rem = lane - i * (S::CPAIR * S::RSEG);
        const int cp = rem / S::RSEG, h0 = (rem - cp * S::RSEG) * S::RLEN;
        float w9[9];
#pragma unroll
        for (int q = 0; q < 9; ++q) w9[q] = a.mixw[pos.c * 9 + q];
        // plane column of image column 2 cp - 2 (the word holding columns 2cp-1 .. 2cp+2 starts
        // one pixel earlier, at an even plane column)
        const uint32_t* zr = (const uint32_t*)(zst + i * S::ZPLANE + 2 * cp);
        // win[a][0..3] = z(h + a - 1, 2cp - 1 .. 2cp + 2): words 0..2 hold columns 2cp-2 .. 2cp+3
        auto row = [&](int hp, float (&r4)[4]) {  // hp: plane row
          const uint32_t w0 = zr[hp * (S::ZP / 2)], w1 = zr[hp * (S::ZP / 2) + 1],
                         w2 = zr[hp * (S::ZP / 2) + 2];
          r4[0] = __uint_as_float(w0 & 0xffff0000u);
          r4[1] = __uint_as_float(w1 << 16);
          r4[2] = __uint_as_float(w1 & 0xffff0000u);
          r4[3] = __uint_as_float(w2 << 16);
        };
        float win[3][4];
        row(h0, win[0]);
        row(h0 + 1, win[1]);
        const int ii = wave * S::IPW + i;  // image of the unit (past the batch: not stored)
        const bool real = ii < pos.nimg;
        uint16_t* yrow = a.y + ((size_t)(pos.img0 + (real ? ii : 0)) * a.C + pos.c) * S::PLANE + 2 * cp;
#pragma unroll 4
        for (int h = h0; h < h0 + S::RLEN; ++h) {
          row(h + 2, win[2]);
          float y0 = 0.f, y1 = 0.f;
#pragma unroll
          for (int u = 0; u < 3; ++u)
#pragma unroll
            for (int t = 0; t < 3; ++t) {
              y0 = fmaf(w9[u * 3 + t], win[u][t], y0);
              y1 = fmaf(w9[u * 3 + t], win[u][t + 1], y1);
            }
          if (real)
            *(uint32_t*)(yrow + (size_t)h * S::IW) =
                __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{y0, y1}), v2bf));
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            win[0][t] = win[1][t];
            win[1][t] = win[2][t];
          }
        }
      }
      wave_lds_sync();  // the planes are read before the next unit's tiles overwrite them
    }
    if constexpr (MORE) convert(conv);
    return nxt;
  };
  constexpr std::true_type kMore{};
  constexpr std::false_type kLast{};

  u32x4 raw[7];
  UnitPos p = unit_pos(a, u0, IPU);
  issue(p, raw);
  convert(raw);
  for (int u = u0; u + 1 < u1; ++u) p = unit(kMore, p, u + 1, raw, raw);
  unit(kLast, p, u1, raw, raw);
}


// ---------------------------------------------------------------------------------- w = 7
// w = 7 on 56x56 images: 64 windows per image, 49 pixels per window. A wave takes one whole
// image of a unit (the 4 waves of a workgroup take 4 consecutive images of a channel) as 4
// wave-units of 16 windows (two window rows). Window rows are padded to 8 pixels, so K = 64 is
// 2 steps of 32 and lane group g feeds window row 4s + g at step s (row 7 is padding, zero).
// Output tiles are two window rows: MFMA rows 0..7 are pixels 0, 1, 2, 3, 3, 4, 5, 6 of row 2t,
// rows 8..15 the same of row 2t + 1 (row 7 of the last tile repeats row 6), so a lane's four
// accumulators are 4 consecutive pixels of one window row, stored as one 8-byte store (pixel 3
// twice, same value). The table operand of the 4 tiles x 2 steps is the same for every window:
// 8 registers of 16 bytes read from the staged table once per channel, so the steady state uses
// no LDS at all.
template <int IW_>
struct Bf7Shape {
  static constexpr int WS = 7, IH = IW_, IW = IW_;
  static constexpr int L1 = 2 * WS - 1;
  static constexpr int PLANE = IH * IW;
  static constexpr int IPW = 1;                    // images per wave (per unit)
  static constexpr int TP = 16;                    // padded table row pitch
  static constexpr int PT = L1 * TP;               // padded table entries
  static constexpr int CS = 240;                   // bf16 per shifted copy
  static constexpr int C0 = PT - 1 - (WS - 1) * TP - (WS - 1);
  static_assert(IW == 56, "shape");
  // the last entry any table run reads (pixel (0, 0), window row 7, shift 7) lies within what
  // stage_table writes
  static_assert(CS % 8 == 0 && C0 + TP * 7 + 7 + 7 <= CS - 8, "copies");
};

template <class S, bool ZS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWgPerCu, 8)))
k_fwd_bf16_w7(BfArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_h[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  uint16_t* copies = smem_h;  // [8][CS]
  const int units = a.C * a.groups;
  const int u0 = (int)((long long)blockIdx.x * units / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * units / gridDim.x);
  if (u0 >= u1) return;  // uniform over the workgroup
  constexpr int IPU = 4 * S::IPW;

  // lane (n, g): MFMA column n = window (n >> 3, n & 7) of the wave-unit's two window rows, MFMA
  // row n = pixel slot n of the tile; lane group g = K block (window row 4s + g) and output slots
  // 4g .. 4g + 3 = window row 2t + (g >> 1), pixels 3 (g & 1) .. + 3
  const int n = lane & 15, g = lane >> 4;
  const int wyl = n >> 3, wx = n & 7;
  // window rows start at 14-byte offsets: load 16 bytes from the 4-byte-aligned pixel
  // 7wx - (wx & 1) (inside the image row) and shift odd windows down by one pixel
  const bool odd = (wx & 1) != 0;
  const int px0 = 7 * wx - (wx & 1);
  const int xo0 = (7 * wyl + g) * S::IW + px0;
  const int xo1 = (7 * wyl + min(4 + g, S::WS - 1)) * S::IW + px0;  // row 7: padding
  const bool pad1 = g == 3;
  const int so = (7 * wyl + (g >> 1)) * S::IW + 7 * wx + 3 * (g & 1);  // tiles t < 3: + 2t rows
  const int so3 = (7 * wyl + S::WS - 1) * S::IW + 7 * wx + 3 * (g & 1);  // tile 3: row 6
  const int xs = n & 7, xi = xs < 4 ? xs : xs - 1;
  const int im = wave * S::IPW;

  auto plane = [&](const UnitPos& p) {
    const int ic = min(im, p.nimg - 1);  // images past the batch read and write its last image
    return ((size_t)(p.img0 + ic) * a.C + p.c) * S::PLANE;
  };
  u32x4 raw[4][2];
  auto issue = [&](const UnitPos& p, int q) {
    const uint16_t* src = a.x + plane(p) + 2 * S::WS * q * S::IW;
    raw[q][0] = *(const u32x4a*)(src + xo0);
    raw[q][1] = *(const u32x4a*)(src + xo1);
  };
  auto operand = [&](const u32x4& in, bool zero) {
    u32x4 o;
    o.x = odd ? __builtin_amdgcn_alignbyte(in.y, in.x, 2) : in.x;
    o.y = odd ? __builtin_amdgcn_alignbyte(in.z, in.y, 2) : in.y;
    o.z = odd ? __builtin_amdgcn_alignbyte(in.w, in.z, 2) : in.z;
    o.w = odd ? in.w >> 16 : in.w & 0xffffu;  // pixel slot 7 is padding
    if (zero) o = u32x4{0u, 0u, 0u, 0u};
    return o;
  };

  u32x4 mvr[4][2];
  int table_c = -1;
  auto unit = [&](auto more, const UnitPos& pos, int u_next) {
    constexpr bool MORE = decltype(more)::value;
    if (pos.c != table_c) {  // uniform over the workgroup
      stage_table<S>(copies, a.T, pos.c);
      table_c = pos.c;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int yi = min(2 * t + (n >> 3), S::WS - 1);
        const int bi = S::C0 - S::TP * yi - xi;
        const int rc = (-bi) & 7;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          mvr[t][s2] = *(const u32x4*)(copies + rc * S::CS + bi + rc + S::TP * (4 * s2 + g));
      }
    }
    const UnitPos nxt = unit_pos(a, u_next < u1 ? u_next : u1 - 1, IPU);
    const size_t obase = plane(pos);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 op0 = operand(raw[q][0], false), op1 = operand(raw[q][1], pad1);
      if constexpr (MORE) issue(nxt, q);  // wave-unit q of the next unit
      v4f acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[t] = mfma_bf16(mvr[t][0], op0, v4f{0.f, 0.f, 0.f, 0.f});
        acc[t] = mfma_bf16(mvr[t][1], op1, acc[t]);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{acc[t][0], acc[t][1]}), v2bf));
        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{acc[t][2], acc[t][3]}), v2bf));
        const size_t o = obase + 2 * S::WS * q * S::IW + (t < 3 ? so + 2 * t * S::IW : so3);
        *(u32x2a2*)(a.y + o) = u32x2a2{lo, hi};
        if constexpr (ZS) *(u32x2a2*)(a.z + o) = u32x2a2{lo, hi};
      }
    }
    return nxt;
  };
  constexpr std::true_type kMore{};
  constexpr std::false_type kLast{};

  UnitPos p = unit_pos(a, u0, IPU);
#pragma unroll
  for (int q = 0; q < 4; ++q) issue(p, q);
  for (int u = u0; u + 1 < u1; ++u) p = unit(kMore, p, u + 1);
  unit(kLast, p, u1);
}

// --------------------------------------------------------------------------------- w = 28
// w = 28 on 56x56 images: 4 windows of 784 pixels per image, so a channel is a 784 x 784 by
// 784 x (4B) product and the work is matrix-bound. A workgroup of 4 waves takes a block of 32
// windows (8 images) of one channel and computes all 784 output pixels for them with
// v_mfma_f32_32x32x16_bf16 (32 pixels x 32 windows x 16 K per instruction); two workgroups run
// per CU, so one's end-of-block store burst overlaps the other's matrix work:
//   * output tiles are window rows (32 MFMA rows: pixels 0..27, then 24..27 again), 28 tiles;
//     wave k owns window rows 7k .. 7k+6: 7 accumulators of 16 registers;
//   * K is walked window row by window row (rows padded to 32 pixels: 2 K steps of 16);
//   * table operand: the staged, reversed, shifted table copies (pitch 64), one aligned 16-byte
//     LDS read per operand; the matrix is block Toeplitz in window rows, so a wave's 7 row
//     tiles need only one new table operand per K step (2 LDS reads per 7 MFMAs);
//   * window operand: window rows stream through a double-buffered LDS chunk (2 window rows of
//     the 32 windows, rows padded with zeros) with one 16-byte load and LDS write per thread and
//     chunk; the loads run PF = 7 chunks ahead; one LDS read per K step;
//   * accumulators hold 4 consecutive pixels of a window row per lane; swapping lane groups
//     between the wave halves (v_permlane32_swap) makes that 8 + 8 pixels: two 16-byte stores
//     per lane and tile.
template <int IW_>
struct Bf28Shape {
  static constexpr int WS = 28, IH = IW_, IW = IW_;
  static constexpr int L1 = 2 * WS - 1;
  static constexpr int PLANE = IH * IW;
  static constexpr int TP = 64;                    // padded table row pitch
  static constexpr int PT = L1 * TP;
  static constexpr int CS = 3544;
  static constexpr int C0 = PT - 1 - (WS - 1) * TP - (WS - 1);
  static constexpr int NWB = 32;                   // windows per block (8 images)
  static constexpr int IPB = NWB / 4;              // images per block
  static constexpr int RC = 2;                     // window rows per chunk
  static constexpr int NCH = WS / RC;              // chunks
  static constexpr int XWP = RC * 32 + 8;          // bf16 per window in a chunk buffer (+16 B)
  static constexpr int XBUF = NWB * XWP;           // bf16 per chunk buffer
  static constexpr int NTH = 256;                  // threads per workgroup (two per CU)
  static constexpr int LPT = NWB * RC * 4 / NTH;   // 16-byte chunk loads per thread
  static constexpr int PF = 7;                     // chunks in flight
  static constexpr int NT = WS / 4;                // output row tiles per wave
  static constexpr int NCT = NWB / 32;             // window tiles
  static_assert(NCT == 1 && NCH % PF == 0 && NCH % 2 == 0, "block shape");
  static_assert(IW == 56, "shape");
  // the last entry a table run reads (pixel (0, 0), window row 27, pixels 24..31, shift 7)
  static_assert(CS % 8 == 0 && C0 + TP * (WS - 1) + 24 + 7 + 7 <= CS - 8, "copies");
  static_assert(NWB * RC * 4 == LPT * NTH, "chunk loads per thread");
  static_assert(NCH >= PF, "chunk ring");
};

template <class S>
constexpr int bf28_lds_bytes() { return (8 * S::CS + 2 * S::XBUF) * 2; }

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) .. f(integral_constant<int, N-1>), in order
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32_bf16(u32x4 a, u32x4 b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

template <class S, bool ZS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_fwd_bf16_w28(BfArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_h[];
  uint16_t* copies = smem_h;                  // [8][CS]
  uint16_t* xbuf = smem_h + 8 * S::CS;        // [2][NWB][XWP]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // persistent: workgroup g walks the blocks [g nb / grid, (g+1) nb / grid); consecutive blocks
  // mostly share a channel (the table is restaged only when it changes) and the window chunks
  // run PF ahead across block boundaries
  const int nb = a.C * a.groups;
  const int b0 = (int)((long long)blockIdx.x * nb / gridDim.x);
  const int b1 = (int)((long long)(blockIdx.x + 1) * nb / gridDim.x);
  if (b0 >= b1) return;  // uniform over the workgroup
  struct Blk {
    int c, img0, nimg;
  };
  auto blk = [&](int b) {
    Blk k;
    k.c = b / a.groups;
    k.img0 = (b - k.c * a.groups) * S::IPB;
    k.nimg = min(a.B - k.img0, S::IPB);
    return k;
  };
  // element offset of the plane of image im of block k (images past the batch read and write its
  // last image: same values)
  auto plane = [&](const Blk& k, int im) {
    return ((size_t)(k.img0 + min(im, k.nimg - 1)) * a.C + k.c) * S::PLANE;
  };

  // chunk loads: thread -> window jw, chunk row r, 8-pixel segment k (segment 3 loads pixels
  // 20..27 and keeps 24..27, padding 28..31 with zeros, so no load leaves the window row)
  static_assert(S::LPT == 1, "one chunk load per thread");
  const int jw = threadIdx.x >> 3, r_ld = (threadIdx.x >> 2) & 1, k_ld = threadIdx.x & 3;
  const int ld_off = (S::WS * ((jw >> 1) & 1) + r_ld) * S::IW + S::WS * (jw & 1) + (k_ld < 3 ? 8 * k_ld : 20);
  const int st_off = jw * S::XWP + r_ld * 32 + 8 * k_ld;
  auto ld_base = [&](const Blk& k) { return plane(k, jw >> 2) + ld_off; };
  auto load_chunk = [&](size_t base, int ch) {
    return *(const u32x4a*)(a.x + base + (size_t)(S::RC * ch) * S::IW);
  };
  auto store_chunk = [&](const u32x4& v, int buf) {
    // the segment test is made opaque here, so the compiler cannot move the select (and with it
    // a wait for the load) up to where the load was issued
    const bool s3 = opaque(k_ld) == 3;
    const u32x4 w = s3 ? u32x4{v.z, v.w, 0u, 0u} : v;
    *(u32x4*)(xbuf + buf * S::XBUF + st_off) = w;
  };

  Blk cur = blk(b0);
  size_t base_cur = ld_base(cur);
  int table_c = cur.c;
  u32x4 pre[S::PF];  // chunk k of the stream in slot k % PF
  {
    TableStage<S, S::NTH> ts;
    ts.load(a.T, cur.c);  // before the pixel loads: waiting for it never waits for them
#pragma unroll
    for (int k = 0; k < S::PF; ++k) {
      pre[k] = load_chunk(base_cur, k);
      __builtin_amdgcn_sched_barrier(0);  // in chunk order: chunk 0's wait is then the shortest
    }
    ts.write(copies);  // ends with a barrier
  }
  store_chunk(pre[0], 0);
  __syncthreads();

  // lane (l32, kh): MFMA row l32 = pixel slot, column l32 = window of the tile, K half kh
  const int l32 = lane & 31, kh = lane >> 5;
  const int xi = l32 < S::WS ? l32 : l32 - 4;  // slots 28..31 repeat pixels 24..27
  const int bi0 = S::C0 - xi;
  const int rc = (-bi0) & 7;
  const int t0 = S::NT * wave;                 // first window row (output tile) of this wave
  // table run of output row yi, K window row yk, K half hs: ab + TP (yk - yi) + 16 hs
  const int ab = rc * S::CS + bi0 + rc + 8 * kh - S::TP * t0;
  const int xb = l32 * S::XWP + 8 * kh;

  for (int b = b0; b < b1; ++b) {
    const Blk nxt = blk(b + 1 < b1 ? b + 1 : b);  // the last block's lookahead re-reads itself
    const size_t base_nxt = ld_base(nxt);
    if (cur.c != table_c) {  // uniform; every wave is past the previous block's last chunk
      stage_table<S, S::NTH>(copies, a.T, cur.c);
      table_c = cur.c;
    }
    v16f acc[S::NT];
#pragma unroll
    for (int t = 0; t < S::NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
    // The table operand of output row yi and K window row yk depends only on d = yk - yi (the
    // matrix is block Toeplitz in window rows): wave rows t0 + t, t < NT, at K row yk use
    // d - d0 = yk - t with d0 = -t0, so at each K row only tile 0 needs a new operand and the
    // other tiles take over the operand tile t - 1 used one K row earlier. With the K loop fully
    // unrolled these are plain registers: areg[yk - t + NT - 1][hs], each live for NT K rows.
    u32x4 areg[S::WS + S::NT - 1][2];
    // chunk ch sits in register slot ch % PF and LDS buffer ch % 2 (NCH is a multiple of both):
    // its slot is free once it is in LDS, so chunk ch + PF of the stream (of this block or the
    // next) goes in flight there; at the end chunk ch + 1 is written to the other buffer
    static_for<S::NCH>([&](auto chc) {
      constexpr int CH = decltype(chc)::value, SL = CH % S::PF, BUF = CH % 2;
      pre[SL] = CH + S::PF < S::NCH ? load_chunk(base_cur, CH + S::PF)
                                    : load_chunk(base_nxt, CH + S::PF - S::NCH);
      const uint16_t* xs = xbuf + BUF * S::XBUF + xb;
#pragma unroll
      for (int r = 0; r < S::RC; ++r)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const int yk = S::RC * CH + r;
          const u32x4 bv = *(const u32x4*)(xs + r * 32 + 16 * hs);
#pragma unroll
          for (int t = 0; t < S::NT; ++t)
            if (t == 0 || yk == 0)  // first use of d = yk - t
              areg[yk - t + S::NT - 1][hs] = *(const u32x4*)(copies + ab + S::TP * (yk - t) + 16 * hs);
#pragma unroll
          for (int t = 0; t < S::NT; ++t)
            acc[t] = mfma32_bf16(areg[yk - t + S::NT - 1][hs], bv, acc[t]);
        }
      // chunk ch + 1 into the other buffer (every wave is past chunk ch - 1, which used it)
      store_chunk(pre[(SL + 1) % S::PF], BUF ^ 1);
      __syncthreads();
    });
    // stores: lane (window l32, kh) holds rows 8g + 4kh .. +3 = 4 consecutive pixels of its
    // window row (group 3 of the upper half repeats pixels 24..27). Swapping groups between lane
    // halves (v_permlane32_swap) gives the lower lanes pixels 0..7 and 16..23 and the upper
    // lanes 8..15 and 20..27 (20..23 also stored by the lower lanes, same values): two 16-byte
    // stores per tile.
    {
      const int j = l32;
      const size_t ob = plane(cur, j >> 2) + (size_t)(S::WS * ((j >> 1) & 1) + t0) * S::IW + S::WS * (j & 1);
      const size_t o1 = ob + (kh ? 8 : 0), o2 = ob + (kh ? 20 : 16);
#pragma unroll
      for (int t = 0; t < S::NT; ++t) {
        const v16f& d = acc[t];
        uint32_t pk[8];  // group g: pk[2g], pk[2g + 1]
#pragma unroll
        for (int q = 0; q < 8; ++q)
          pk[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{d[2 * q], d[2 * q + 1]}), v2bf));
        const uint32_t g2lo = pk[4], g2hi = pk[5];
        // (group 0, group 1) and (group 2, group 3): lower lanes receive the upper lanes' first
        // group, upper lanes the lower lanes' second group
        auto sw01a = __builtin_amdgcn_permlane32_swap(pk[0], pk[2], false, false);
        auto sw01b = __builtin_amdgcn_permlane32_swap(pk[1], pk[3], false, false);
        auto sw23a = __builtin_amdgcn_permlane32_swap(pk[4], pk[6], false, false);
        auto sw23b = __builtin_amdgcn_permlane32_swap(pk[5], pk[7], false, false);
        const u32x4 v1 = u32x4{sw01a[0], sw01b[0], sw01a[1], sw01b[1]};
        const u32x4 v2 = kh ? u32x4{g2lo, g2hi, sw23a[0], sw23b[0]} : u32x4{sw23a[0], sw23b[0], sw23a[1], sw23b[1]};
        *(u32x4a*)(a.y + o1 + (size_t)t * S::IW) = v1;
        *(u32x4a*)(a.y + o2 + (size_t)t * S::IW) = v2;
        if constexpr (ZS) {
          *(u32x4a*)(a.z + o1 + (size_t)t * S::IW) = v1;
          *(u32x4a*)(a.z + o2 + (size_t)t * S::IW) = v2;
        }
      }
    }
    cur = nxt;
    base_cur = base_nxt;
  }
}

enum BfShapeId { BF_NONE, BF_28, BF_56, BF7_56, BF28_56 };

BfShapeId bf_shape(const FwdRequest& r) {
  if (r.layout != 0 || r.H != r.W) return BF_NONE;
  if (r.w == 14 && r.H == 28) return BF_28;
  if (r.w == 14 && r.H == 56) return BF_56;
  if (r.w == 7 && r.H == 56) return BF7_56;
  if (r.w == 28 && r.H == 56) return BF28_56;
  return BF_NONE;
}

constexpr int kLdsPerCu = 160 * 1024, kLdsGranule = 1280;
constexpr bool fits(int bytes) {
  return (bytes + kLdsGranule - 1) / kLdsGranule * kLdsGranule * kWgPerCu <= kLdsPerCu;
}
static_assert(fits(bf_lds_bytes<BfShape<28>>()) && fits(bf_lds_bytes<BfShape<56>>()) &&
                  fits(bf_lds_bytes<Bf7Shape<56>>()),
              "resident workgroups per CU");

static_assert((bf_mix_lds_bytes<BfShape<28>>() + kLdsGranule - 1) / kLdsGranule * kLdsGranule *
                      kWgPerCuMix <= kLdsPerCu &&
                  (bf_mix_lds_bytes<BfShape<56>>() + kLdsGranule - 1) / kLdsGranule * kLdsGranule *
                      kWgPerCuMix <= kLdsPerCu,
              "resident workgroups per CU with the fused mix");

template <class S, bool MIX = false, class K>
hipError_t launch_bf(const FwdRequest& r, hipStream_t st, K with_z, K without_z) {
  BfArgs a{};
  a.B = r.B;
  a.C = r.C;
  a.groups = (r.B + 4 * S::IPW - 1) / (4 * S::IPW);
  a.x = (const uint16_t*)r.x;
  a.T = (const uint16_t*)r.T;
  a.y = (uint16_t*)r.y;
  a.z = (uint16_t*)r.zsave;
  a.mixw = MIX ? r.mixw : nullptr;
  int lds;
  if constexpr (MIX) lds = bf_mix_lds_bytes<S>();
  else lds = bf_lds_bytes<S>();
  const int per_cu = MIX ? kWgPerCuMix : kWgPerCu;
  const K fn = a.z ? with_z : without_z;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int units = a.C * a.groups;
  const int grid = units < per_cu * cus ? units : per_cu * cus;
  return launch_main(fn, dim3(grid), dim3(kThreads), lds, st, a);
}

// Persistent workgroups of 4 waves, two per CU, each walking a run of blocks of 32 windows.
template <class S>
hipError_t launch_bf28(const FwdRequest& r, hipStream_t st) {
  BfArgs a{};
  a.B = r.B;
  a.C = r.C;
  a.groups = (r.B + S::IPB - 1) / S::IPB;
  a.x = (const uint16_t*)r.x;
  a.T = (const uint16_t*)r.T;
  a.y = (uint16_t*)r.y;
  a.z = (uint16_t*)r.zsave;
  const int lds = bf28_lds_bytes<S>();
  auto fn = a.z ? k_fwd_bf16_w28<S, true> : k_fwd_bf16_w28<S, false>;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int nb = a.C * a.groups;
  const int grid = nb < 2 * cus ? nb : 2 * cus;  // two resident workgroups per CU
  return launch_main(fn, dim3(grid), dim3(S::NTH), lds, st, a);
}
static_assert(2 * ((bf28_lds_bytes<Bf28Shape<56>>() + kLdsGranule - 1) / kLdsGranule * kLdsGranule) <=
                  kLdsPerCu,
              "two w = 28 workgroups per CU");

}  // namespace

// bf16 maps with the 3x3 mix, w = 14 on 28x28 / 56x56 images: the mix fused into the fast
// forward (y and z_save bf16).
bool fast_bf16_fused_mix_ok(const FwdRequest& r) {
  if (!r.mixw) return false;
  FwdRequest q = r;
  q.mixw = nullptr;
  return fast_bf16_forward_ok(q) && (bf_shape(q) == BF_28 || bf_shape(q) == BF_56);
}

hipError_t launch_forward_fast_bf16_mix(const FwdRequest& r, hipStream_t st) {
  switch (bf_shape(r)) {
    case BF_28:
      return launch_bf<BfShape<28>, true>(r, st, k_fwd_bf16<BfShape<28>, true, false, true>,
                                          k_fwd_bf16<BfShape<28>, false, false, true>);
    case BF_56:
      return launch_bf<BfShape<56>, true>(r, st, k_fwd_bf16<BfShape<56>, true, false, true>,
                                          k_fwd_bf16<BfShape<56>, false, false, true>);
    default: return hipErrorInvalidValue;
  }
}

bool fast_bf16_forward_ok(const FwdRequest& r) {
  // unit indices (C * groups) are ints
  return r.in_bf16 && r.out_bf16 && r.T && !r.M && !r.mixw && !r.Tsub && r.oy == 0 &&
         r.ox == 0 && r.B > 0 && r.C > 0 &&
         (long long)r.C * ((r.B + 3) / 4 + 1) < ((long long)1 << 31) && bf_shape(r) != BF_NONE;
}

// dX = M_c^T G_c of the bf16 backward (w = 14, NCHW 28x28 or 56x56 images): the forward
// contraction on G with the table staged rotated, written as bf16.
hipError_t launch_bf16_transposed_contraction(const uint16_t* g, const uint16_t* T, uint16_t* out,
                                              int B, int C, int H, hipStream_t st) {
  FwdRequest r{};
  r.B = B; r.C = C; r.H = H; r.W = H; r.w = 14; r.layout = 0;
  r.in_bf16 = 1; r.out_bf16 = 1;
  r.x = g; r.T = T; r.y = out;
  switch (bf_shape(r)) {
    case BF_28: return launch_bf<BfShape<28>>(r, st, k_fwd_bf16<BfShape<28>, false, true>, k_fwd_bf16<BfShape<28>, false, true>);
    case BF_56: return launch_bf<BfShape<56>>(r, st, k_fwd_bf16<BfShape<56>, false, true>, k_fwd_bf16<BfShape<56>, false, true>);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward_fast_bf16(const FwdRequest& r, hipStream_t st) {
  switch (bf_shape(r)) {
    case BF_28: return launch_bf<BfShape<28>>(r, st, k_fwd_bf16<BfShape<28>, true>, k_fwd_bf16<BfShape<28>, false>);
    case BF_56: return launch_bf<BfShape<56>>(r, st, k_fwd_bf16<BfShape<56>, true>, k_fwd_bf16<BfShape<56>, false>);
    case BF7_56:
      return launch_bf<Bf7Shape<56>>(r, st, k_fwd_bf16_w7<Bf7Shape<56>, true>, k_fwd_bf16_w7<Bf7Shape<56>, false>);
    case BF28_56: return launch_bf28<Bf28Shape<56>>(r, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wbmm

// CPU check of the FFT gray-block arithmetic of the HIP path (fi_fft.h compiled for the host):
// one transform team is emulated thread by thread, group by group, exactly in the order the
// kernel runs, and the result is compared with the direct sum of the gray block.
#include <cmath>
#include <cstdio>
#include <random>
#include <vector>
#include "../../long_convolution_sequence_amd/csrc/fi_fft.h"
using namespace fi;
// Emulate one transform team of the tile kernel sequentially (thread by thread per group).
template <int LOGN> struct Emu {
  using S = FftShape<LOGN>;
  static constexpr int N = S::N, TT = S::TT, R0 = S::R0, QLOG0 = S::QLOG0, HALF0 = S::HALF0;
  template <int PASS, bool FWD> static void groups(std::vector<float2>& X, const float2* tw, int logNT) {
    if constexpr (FWD) { if constexpr (PASS < S::NPASS) { for (int lt = 0; lt < TT; ++lt) lds_group<LOGN, PASS, true>(X.data(), lt, tw, logNT); groups<PASS + 1, true>(X, tw, logNT); } }
    else { if constexpr (PASS >= 1) { for (int lt = 0; lt < TT; ++lt) lds_group<LOGN, PASS, false>(X.data(), lt, tw, logNT); groups<PASS - 1, false>(X, tw, logNT); } }
  }
  // forward transform of 2N reals src (pruned: upper half zero) -> X (bit reversed, LDS layout)
  static void forward(const float* src, bool pruned, std::vector<float2>& X, const float2* tw, int logNT) {
    X.assign(lds_len(N), make_float2(0, 0));
    const float2* s2 = reinterpret_cast<const float2*>(src);
    for (int lt = 0; lt < TT; ++lt) {
      float2 v[1 << R0];
      for (int m = 0; m < (1 << R0); ++m) v[m] = (pruned && m >= HALF0) ? make_float2(0, 0) : s2[lt + (m << QLOG0)];
      if (pruned) dif_group<R0, true>(v, lt, LOGN, tw, logNT); else dif_group<R0>(v, lt, LOGN, tw, logNT);
      for (int m = 0; m < (1 << R0); ++m) X[lpad(lt + (m << QLOG0))] = v[m];
    }
    groups<1, true>(X, tw, logNT);
  }
  static void spectrum(const float* g, std::vector<float4>& spec, const float2* tw, int logNT) {
    std::vector<float2> X; forward(g, false, X, tw, logNT);
    spec.resize(N / 2); const float inv = 1.0f / N;
    for (int j = 0; j < N / 2; ++j) {
      if (j == 0) { float2 C0 = X[0], Ch = X[lpad(1)]; spec[0] = make_float4((C0.x + C0.y) * inv, (C0.x - C0.y) * inv, Ch.x * inv, -Ch.y * inv); }
      else { float2 A1, A2; real_bins(X[lpad(bitrev<LOGN>(j))], X[lpad(bitrev<LOGN>(N - j))], twiddle(tw, logNT, LOGN + 1, j), A1, A2);
             spec[j] = make_float4(A1.x * inv, A1.y * inv, A2.x * inv, A2.y * inv); }
    }
  }
  static void tile(const float* x, const std::vector<float4>& sp, float* acc, const float2* tw, int logNT) {
    std::vector<float2> X; forward(x, true, X, tw, logNT);
    for (int j = 0; j < N / 2; ++j) {
      float4 g = sp[j];
      if (j == 0) { float2 C0 = X[0], Ch = X[lpad(1)]; float Z0 = (C0.x + C0.y) * g.x, ZN = (C0.x - C0.y) * g.y;
        X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN)); X[lpad(1)] = cmulc(Ch, make_float2(g.z, g.w)); }
      else { int p1 = lpad(bitrev<LOGN>(j)), p2 = lpad(bitrev<LOGN>(N - j)); float2 W = twiddle(tw, logNT, LOGN + 1, j);
        float2 A1, A2, D1, D2; real_bins(X[p1], X[p2], W, A1, A2);
        pack_inverse(cmul(A1, make_float2(g.x, g.y)), cmul(A2, make_float2(g.z, g.w)), W, D1, D2); X[p1] = D1; X[p2] = D2; }
    }
    groups<S::NPASS - 1, false>(X, tw, logNT);
    float2* a2 = reinterpret_cast<float2*>(acc);
    for (int lt = 0; lt < TT; ++lt) {
      float2 v[1 << R0];
      for (int m = 0; m < (1 << R0); ++m) v[m] = X[lpad(lt + (m << QLOG0))];
      dit_group<R0>(v, lt, LOGN, tw, logNT);
      for (int m = 0; m < HALF0; ++m) a2[lt + (m << QLOG0)] = cadd(a2[lt + (m << QLOG0)], v[m + HALF0]);
    }
  }
};
template <int LOGN> double run(int logNT) {
  const int U = 1 << LOGN, NT = 1 << logNT;
  std::vector<float2> tw(NT);
  for (int k = 0; k < NT; ++k) { double a = -2.0 * M_PI * k / NT; tw[k] = make_float2((float)cos(a), (float)sin(a)); }
  std::mt19937 rng(LOGN); std::normal_distribution<float> nd;
  std::vector<float> h(2 * U), x(2 * U, 0.f), acc(U);
  for (auto& v : h) v = nd(rng);
  for (int i = 0; i < U; ++i) x[i] = nd(rng);
  for (auto& v : acc) v = nd(rng);
  std::vector<float4> sp; Emu<LOGN>::spectrum(h.data(), sp, tw.data(), logNT);
  std::vector<float> out = acc; Emu<LOGN>::tile(x.data(), sp, out.data(), tw.data(), logNT);
  double worst = 0, scale = 0;
  for (int j = 0; j < U; ++j) { // output j (slot t+1+j): sum_k h[j+U-k] x[k]
    double s = acc[j]; double a = 0;
    for (int k = 0; k < U; ++k) { s += (double)h[j + U - k] * x[k]; a += fabs((double)h[j + U - k] * x[k]); }
    worst = std::max(worst, fabs(out[j] - s)); scale = std::max(scale, a);
  }
  return worst / scale;
}
int main() {
  double r[13] = { run<2>(15), run<3>(15), run<4>(15), run<5>(15), run<6>(15), run<7>(15), run<8>(15), run<9>(15), run<10>(15), run<11>(15), run<12>(15), run<13>(15), run<14>(15) };
  int bad = 0;
  for (int i = 0; i < 13; ++i) { printf("LOGN=%d rel err %.3e\n", i + 2, r[i]); if (!(r[i] < 1e-5)) bad = 1; }
  return bad;
}

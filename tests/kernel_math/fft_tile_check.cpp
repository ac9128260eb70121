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
    if constexpr (FWD) { if constexpr (PASS < S::NPASS) { for (int lt = 0; lt < TT; ++lt) lds_group<LOGN, PASS, true>(X.data(), lt, group_root<LOGN, PASS>(lt, tw, logNT)); groups<PASS + 1, true>(X, tw, logNT); } }
    else { if constexpr (PASS >= 1) { for (int lt = 0; lt < TT; ++lt) lds_group<LOGN, PASS, false>(X.data(), lt, group_root<LOGN, PASS>(lt, tw, logNT)); groups<PASS - 1, false>(X, tw, logNT); } }
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
  // ptw: pair twiddles, W_{2N}^j of item e at ptw[N/2 + e] (as the library's table)
  static void spectrum(const float* g, std::vector<float4>& spec, const float2* tw, const float2* ptw, int logNT) {
    std::vector<float2> X; forward(g, false, X, tw, logNT);
    spec.resize(N / 2); const float inv = 1.0f / N;
    for (int e = 0; e < N / 2; ++e) {
      if (e == 0) { float2 C0 = X[0], Ch = X[lpad(1)]; spec[0] = make_float4((C0.x + C0.y) * inv, (C0.x - C0.y) * inv, Ch.x * inv, -Ch.y * inv); }
      else { PairSlot ps = pair_slot(LOGN, e); float2 A1, A2; real_bins(X[lpad(ps.pj)], X[lpad(ps.pm)], ptw[N / 2 + e], A1, A2);
             spec[e] = make_float4(A1.x * inv, A1.y * inv, A2.x * inv, A2.y * inv); }
    }
  }
  static void tile(const float* x, const std::vector<float4>& sp, float* acc, const float2* tw, const float2* ptw, int logNT) {
    std::vector<float2> X; forward(x, true, X, tw, logNT);
    for (int e = 0; e < N / 2; ++e) {
      float4 g = sp[e];
      if (e == 0) { float2 C0 = X[0], Ch = X[lpad(1)]; float Z0 = (C0.x + C0.y) * g.x, ZN = (C0.x - C0.y) * g.y;
        X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN)); X[lpad(1)] = cmulc(Ch, make_float2(g.z, g.w)); }
      else { PairSlot ps = pair_slot(LOGN, e); int p1 = lpad(ps.pj), p2 = lpad(ps.pm); float2 W = ptw[N / 2 + e];
        float2 A1, A2, D1, D2; real_bins(X[p1], X[p2], W, A1, A2);
        pack_inverse(cmul(A1, make_float2(g.x, g.y)), cmul(A2, make_float2(g.z, g.w)), W, D1, D2); X[p1] = D1; X[p2] = D2; }
    }
    groups<S::NPASS - 1, false>(X, tw, logNT);
    float2* a2 = reinterpret_cast<float2*>(acc);
    for (int lt = 0; lt < TT; ++lt) {
      float2 v[1 << R0];
      for (int m = 0; m < (1 << R0); ++m) v[m] = X[lpad(lt + (m << QLOG0))];
      dit_group_w<R0>(v, group_root<LOGN, 0>(lt, tw, logNT));
      for (int m = 0; m < HALF0; ++m) a2[lt + (m << QLOG0)] = cadd(a2[lt + (m << QLOG0)], v[m + HALF0]);
    }
  }
};
// The two-half form of a 2M-point gray block (k_fft_tile2 / k_spectrum2): the
// U = 2M point complex transform as its odd-bin and even-bin M-point halves.
template <int LOGM> struct Emu2 {
  using E = Emu<LOGM>;
  static constexpr int M = 1 << LOGM, U = 2 * M, TT = E::TT, R0 = E::R0, QLOG0 = E::QLOG0;
  static float2 w(const float2* tw, int logNT, int slog, int i) { return twiddle(tw, logNT, slog, i); }
  // half input: even: lo + hi; odd: (lo - hi) W_U^i
  static void half_forward(const float2* lo, const float2* hi, bool odd, std::vector<float2>& X, const float2* tw, int logNT) {
    std::vector<float2> in(M);
    for (int i = 0; i < M; ++i) {
      float2 a = lo[i], b = hi ? hi[i] : make_float2(0, 0);
      in[i] = odd ? cmul(csub(a, b), w(tw, logNT, LOGM + 1, i)) : cadd(a, b);
    }
    E::forward(reinterpret_cast<const float*>(in.data()), false, X, tw, logNT);
  }
  static void spectrum(const float* g, std::vector<float4>& spec, const float2* tw, const float2* ptw, const float2* optw, int logNT) {
    const float2* g2 = reinterpret_cast<const float2*>(g);
    spec.assign(M, make_float4(0, 0, 0, 0)); const float inv = 1.0f / U;
    for (int odd = 1; odd >= 0; --odd) {
      std::vector<float2> X; half_forward(g2, g2 + M, odd, X, tw, logNT);
      for (int e = 0; e < M / 2; ++e) {
        if (!odd && e == 0) { float2 C0 = X[0], Ch = X[lpad(1)]; spec[0] = make_float4((C0.x + C0.y) * inv, (C0.x - C0.y) * inv, Ch.x * inv, -Ch.y * inv); continue; }
        PairSlot ps = odd ? odd_slot(LOGM, e) : pair_slot(LOGM, e); float2 A1, A2;
        real_bins(X[lpad(ps.pj)], X[lpad(ps.pm)], (odd ? optw : ptw)[M / 2 + e], A1, A2);
        spec[(odd ? M / 2 : 0) + e] = make_float4(A1.x * inv, A1.y * inv, A2.x * inv, A2.y * inv);
      }
    }
  }
  static void tile(const float* x, const std::vector<float4>& sp, float* acc, const float2* tw, const float2* ptw, const float2* optw, int logNT) {
    const float2* x2 = reinterpret_cast<const float2*>(x);
    float2* a2 = reinterpret_cast<float2*>(acc);
    for (int odd = 1; odd >= 0; --odd) {
      std::vector<float2> X; half_forward(x2, nullptr, odd, X, tw, logNT);
      for (int e = 0; e < M / 2; ++e) {
        float4 g = sp[(odd ? M / 2 : 0) + e];
        if (!odd && e == 0) { float2 C0 = X[0], Ch = X[lpad(1)]; float Z0 = (C0.x + C0.y) * g.x, ZN = (C0.x - C0.y) * g.y;
          X[0] = make_float2(0.5f * (Z0 + ZN), 0.5f * (Z0 - ZN)); X[lpad(1)] = cmulc(Ch, make_float2(g.z, g.w)); continue; }
        PairSlot ps = odd ? odd_slot(LOGM, e) : pair_slot(LOGM, e); int p1 = lpad(ps.pj), p2 = lpad(ps.pm);
        float2 W = (odd ? optw : ptw)[M / 2 + e], A1, A2, D1, D2; real_bins(X[p1], X[p2], W, A1, A2);
        pack_inverse(cmul(A1, make_float2(g.x, g.y)), cmul(A2, make_float2(g.z, g.w)), W, D1, D2); X[p1] = D1; X[p2] = D2;
      }
      E::template groups<E::S::NPASS - 1, false>(X, tw, logNT);
      for (int lt = 0; lt < TT; ++lt) {
        float2 v[1 << R0];
        for (int m = 0; m < (1 << R0); ++m) v[m] = X[lpad(lt + (m << QLOG0))];
        dit_group<R0>(v, lt, LOGM, tw, logNT);
        for (int m = 0; m < (1 << R0); ++m) {
          const int i = lt + (m << QLOG0);
          a2[i] = odd ? csub(a2[i], cmulc(v[m], w(tw, logNT, LOGM + 1, i))) : cadd(a2[i], v[m]);
        }
      }
    }
  }
};
template <int LOGM> double run2(int logNT) {
  const int M = 1 << LOGM, U = 2 * M, NT = 1 << logNT;
  std::vector<float2> tw(NT), ptw(M, make_float2(1, 0)), optw(M, make_float2(1, 0));
  for (int k = 0; k < NT; ++k) { double a = -2.0 * M_PI * k / NT; tw[k] = make_float2((float)cos(a), (float)sin(a)); }
  for (int e = 1; e < M / 2; ++e) { double a = -M_PI * pair_slot(LOGM, e).j / M; ptw[M / 2 + e] = make_float2((float)cos(a), (float)sin(a)); }
  for (int e = 0; e < M / 2; ++e) { double a = -M_PI * odd_slot(LOGM, e).j / (2.0 * M); optw[M / 2 + e] = make_float2((float)cos(a), (float)sin(a)); }
  std::mt19937 rng(100 + LOGM); std::normal_distribution<float> nd;
  std::vector<float> h(2 * U), x(U), acc(U);
  for (auto& v : h) v = nd(rng);
  for (auto& v : x) v = nd(rng);
  for (auto& v : acc) v = nd(rng);
  std::vector<float4> sp; Emu2<LOGM>::spectrum(h.data(), sp, tw.data(), ptw.data(), optw.data(), logNT);
  std::vector<float> out = acc; Emu2<LOGM>::tile(x.data(), sp, out.data(), tw.data(), ptw.data(), optw.data(), logNT);
  double worst = 0, scale = 0;
  for (int j = 0; j < U; ++j) {  // output j: sum_k h[j+U-k] x[k]
    double s = acc[j], a = 0;
    for (int k = 0; k < U; ++k) { s += (double)h[j + U - k] * x[k]; a += fabs((double)h[j + U - k] * x[k]); }
    worst = std::max(worst, fabs(out[j] - s)); scale = std::max(scale, a);
  }
  return worst / scale;
}
template <int LOGN> double run(int logNT) {
  const int U = 1 << LOGN, NT = 1 << logNT;
  std::vector<float2> tw(NT), ptw(U, make_float2(1, 0));
  for (int k = 0; k < NT; ++k) { double a = -2.0 * M_PI * k / NT; tw[k] = make_float2((float)cos(a), (float)sin(a)); }
  for (int e = 1; e < U / 2; ++e) { double a = -M_PI * pair_slot(LOGN, e).j / U; ptw[U / 2 + e] = make_float2((float)cos(a), (float)sin(a)); }
  std::mt19937 rng(LOGN); std::normal_distribution<float> nd;
  std::vector<float> h(2 * U), x(2 * U, 0.f), acc(U);
  for (auto& v : h) v = nd(rng);
  for (int i = 0; i < U; ++i) x[i] = nd(rng);
  for (auto& v : acc) v = nd(rng);
  std::vector<float4> sp; Emu<LOGN>::spectrum(h.data(), sp, tw.data(), ptw.data(), logNT);
  std::vector<float> out = acc; Emu<LOGN>::tile(x.data(), sp, out.data(), tw.data(), ptw.data(), logNT);
  double worst = 0, scale = 0;
  for (int j = 0; j < U; ++j) { // output j (slot t+1+j): sum_k h[j+U-k] x[k]
    double s = acc[j]; double a = 0;
    for (int k = 0; k < U; ++k) { s += (double)h[j + U - k] * x[k]; a += fabs((double)h[j + U - k] * x[k]); }
    worst = std::max(worst, fabs(out[j] - s)); scale = std::max(scale, a);
  }
  return worst / scale;
}
// The real-spectrum items: every position exactly once, bins j and N-j at the
// named positions, and (N >= 256) sixteen consecutive items touch sixteen
// distinct LDS bank slots through either position.
static int check_pairs(int logn) {
  const int N = 1 << logn;
  std::vector<int> seen(N, 0);
  int bad = 0;
  for (int e = 0; e < N / 2; ++e) {
    PairSlot ps = pair_slot(logn, e);
    seen[ps.pj]++; seen[ps.pm]++;
    if (e == 0) { bad |= !(ps.pj == 0 && ps.pm == 1 && ps.j == 0); continue; }
    const int kj = rbits(logn, ps.pj), km = rbits(logn, ps.pm);
    bad |= !(kj == ps.j && ps.j > 0 && ps.j < N / 2 && km == N - ps.j);
  }
  for (int i = 0; i < N; ++i) bad |= seen[i] != 1;
  if (logn >= 8)
    for (int e0 = 0; e0 < N / 2; e0 += 16) {
      int mj = 0, mm = 0;
      for (int i = (e0 == 0 ? 1 : 0); i < 16; ++i) {
        PairSlot ps = pair_slot(logn, e0 + i);
        mj |= 1 << (lpad(ps.pj) & 15); mm |= 1 << (lpad(ps.pm) & 15);
      }
      const int want = e0 == 0 ? 15 : 16;
      bad |= __builtin_popcount(mj) != want || __builtin_popcount(mm) != want;
    }
  printf("pairs LOGN=%d %s\n", logn, bad ? "BAD" : "ok");
  return bad;
}
// The per-thread form of the pair slots (pair_base / pair_slot_m) against pair_slot for every
// thread and item m >= 1, and for item 0 of the threads lt >= 16.
template <int LOGN> int check_pair_base() {
  const int N = 1 << LOGN, TT = N / 16;
  int bad = 0;
  for (int lt = 0; lt < TT; ++lt) {
    const PairBase b = pair_base<LOGN>(lt);
    for (int m = (lt < 16 ? 1 : 0); m < (N / 2) / TT; ++m) {
      const PairSlot f = pair_slot_m<LOGN>(b, m), r = pair_slot(LOGN, lt + m * TT);
      if (f.pj != r.pj || f.pm != r.pm) ++bad;
    }
  }
  // the padded slots every kernel item uses (item_lds), for every item but e = 0
  const PairLds L = pair_lds<LOGN>(0);
  (void)L;
  for (int lt = 0; lt < TT; ++lt) {
    const PairLds pl = pair_lds<LOGN>(lt);
    for (int m = 0; m < (N / 2) / TT; ++m) {
      if (lt + m * TT == 0) continue;
      const SlotPair f = item_lds<LOGN, N / 16>(pl, lt, m);
      const PairSlot r = pair_slot(LOGN, lt + m * TT);
      if (f.a != lpad(r.pj) || f.b != lpad(r.pm)) ++bad;
    }
  }
  printf("pair base LOGN=%d %s\n", LOGN, bad ? "BAD" : "ok");
  return bad != 0;
}
// item_lds below the per-thread form (N < 256): pair_slot itself
template <int LOGN> int check_small_items() {
  constexpr int N = 1 << LOGN, TT = N >= 16 ? N / 16 : 1;
  int bad = 0;
  for (int lt = 0; lt < TT; ++lt)
    for (int m = 0; m * TT < N / 2; ++m) {
      if (lt + m * TT == 0) continue;
      const SlotPair f = item_lds<LOGN, TT>(pair_lds<LOGN>(lt), lt, m);
      const PairSlot r = pair_slot(LOGN, lt + m * TT);
      if (f.a != lpad(r.pj) || f.b != lpad(r.pm)) ++bad;
    }
  return bad != 0;
}

int main() {
  int pbad = 0;
  for (int logn = 2; logn <= 16; ++logn) pbad |= check_pairs(logn);
  pbad |= check_pair_base<8>() | check_pair_base<9>() | check_pair_base<10>() | check_pair_base<11>() |
          check_pair_base<12>() | check_pair_base<13>() | check_pair_base<14>() | check_pair_base<15>() |
          check_pair_base<16>();
  pbad |= check_small_items<2>() | check_small_items<3>() | check_small_items<4>() | check_small_items<5>() |
          check_small_items<6>() | check_small_items<7>();
  double r[13] = { run<2>(15), run<3>(15), run<4>(15), run<5>(15), run<6>(15), run<7>(15), run<8>(15), run<9>(15), run<10>(15), run<11>(15), run<12>(15), run<13>(15), run<14>(15) };
  int bad = 0;
  for (int i = 0; i < 13; ++i) { printf("LOGN=%d rel err %.3e\n", i + 2, r[i]); if (!(r[i] < 1e-5)) bad = 1; }
  double r2[11] = { run2<2>(15), run2<3>(15), run2<4>(15), run2<5>(15), run2<6>(15), run2<7>(15), run2<8>(15), run2<9>(15), run2<10>(15), run2<12>(15), run2<14>(15) };
  const int l2[11] = {2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 14};
  for (int i = 0; i < 11; ++i) { printf("two halves LOGM=%d rel err %.3e\n", l2[i], r2[i]); if (!(r2[i] < 1e-5)) bad = 1; }
  return bad | pbad;
}

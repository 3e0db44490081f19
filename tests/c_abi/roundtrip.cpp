// roundtrip.cpp -- the C ABI used from C++ alone (no Python): layout, bf16
// and fp8 dispatch, cached dispatch and combine on a small problem; then
// output buffers sized by ep_buffer_size_hint, fp8 dispatch with UE8M0 scales,
// ep_dispatch_noalloc with column-major scales, and fixed-length windows
// (dispatch, status, combine).  Everything is compared byte for byte with the
// CPU oracle (linked from oracle/liboracle.so; test code only).  Exit status 0
// and one "ok" line when everything matches.
//
// Inputs come from a fixed splitmix64 stream: top-k of distinct experts with
// some unused (-1) slots, bf16 rows of moderate magnitude, positive weights.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "ep_mi355x.h"
#include "oracle.h"

namespace {

uint64_t g_state = 0x5EEDu;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int failures = 0;
void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("MISMATCH: %s\n", what);
    ++failures;
  }
}

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      std::printf("HIP error %s at %s\n", hipGetErrorString(e_), #call);          \
      return 2;                                                                   \
    }                                                                             \
  } while (0)
#define EP_OK_(call)                                                              \
  do {                                                                            \
    ep_status s_ = (call);                                                        \
    if (s_ != EP_OK) {                                                            \
      std::printf("ep status %d at %s: %s\n", (int)s_, #call, ep_last_error());    \
      return 3;                                                                   \
    }                                                                             \
  } while (0)

template <typename T>
T* dev_copy(const std::vector<T>& v) {
  T* p = nullptr;
  if (hipMalloc((void**)&p, v.size() * sizeof(T) + 16) != hipSuccess) return nullptr;
  if (!v.empty() && hipMemcpy(p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
  return p;
}

}  // namespace

int main() {
  const int P = 4, S = 50, E = 16, K = 3, H = 256, A = 4;
  const int64_t T = (int64_t)P * S;
  if (ep_abi_version() != EP_ABI_VERSION) {
    std::printf("ABI version %d, header %d\n", ep_abi_version(), EP_ABI_VERSION);
    return 4;
  }

  std::vector<int64_t> topk(T * K);
  for (int64_t u = 0; u < T; ++u) {
    for (int j = 0; j < K; ++j) {
      int64_t e;
      bool dup;
      do {
        e = (int64_t)(next_u64() % E);
        dup = false;
        for (int jj = 0; jj < j; ++jj) dup |= topk[u * K + jj] == e;
      } while (dup);
      topk[u * K + j] = e;
    }
    if (u % 7 == 3) topk[u * K + K - 1] = -1;  // unused slots
  }
  std::vector<uint16_t> x(T * H);
  for (auto& v : x) v = (uint16_t)((next_u64() & 0x807F) | 0x3E00);  // sign, mantissa, exponent near 1
  std::vector<float> w(T * K);
  for (auto& v : w) v = 0.25f + (float)(next_u64() % 1000) / 1000.0f;

  // oracle
  const int El = E / P;
  std::vector<uint8_t> itr(T * P);
  std::vector<int32_t> ntpr(P * P), ntpe(P * E), rpm(P * P), nrecv(P), ne_tot(E), dst_slot(T * K), send_head(T * P),
      recv_src_idx(T * K);
  std::vector<int64_t> eoff(P * (El + 1)), nexp(P), wbase(P + 1), rbase(P + 1);
  if (oracle_layout(P, S, E, K, A, 0, topk.data(), itr.data(), ntpr.data(), ntpe.data(), rpm.data(), nrecv.data(),
                    ne_tot.data(), eoff.data(), nexp.data(), wbase.data(), dst_slot.data(), send_head.data(),
                    recv_src_idx.data(), rbase.data()) != ORACLE_OK)
    return 5;
  const int64_t R = wbase[P];

  // device
  int64_t* d_topk = dev_copy(topk);
  uint16_t* d_x = dev_copy(x);
  float* d_w = dev_copy(w);
  if (!d_topk || !d_x || !d_w) return 2;
  ep_config cfg{P, S, H, K, E, A, 0u, 0};
  ep_handle* h = nullptr;
  int64_t rows = -1;
  EP_OK_(ep_get_layout(&cfg, d_topk, nullptr, &h, &rows));
  expect(rows == R, "total_rows");

  const void* p;
  int64_t n;
  int32_t b;
  EP_OK_(ep_handle_tensor(h, EP_T_DST_SLOT, &p, &n, &b));
  std::vector<int32_t> got_slot(n);
  HIP_OK(hipMemcpy(got_slot.data(), p, n * 4, hipMemcpyDeviceToHost));
  expect(got_slot == dst_slot, "dst_slot");
  EP_OK_(ep_handle_tensor(h, EP_T_SEND_HEAD, &p, &n, &b));
  std::vector<int32_t> got_sh(n);
  HIP_OK(hipMemcpy(got_sh.data(), p, n * 4, hipMemcpyDeviceToHost));
  expect(got_sh == send_head, "send_head");

  for (int fp8 = 0; fp8 < 2; ++fp8) {
    const size_t row_bytes = fp8 ? H : 2 * H;
    void* d_rx;
    float *d_sc, *d_rw;
    int32_t* d_meta;
    HIP_OK(hipMalloc(&d_rx, R * row_bytes + 16));
    HIP_OK(hipMalloc((void**)&d_sc, R * (H / 128) * 4 + 16));
    HIP_OK(hipMalloc((void**)&d_rw, R * 4 + 16));
    HIP_OK(hipMalloc((void**)&d_meta, R * 8 + 16));
    const uint32_t flags = EP_DISPATCH_ZERO_PADDING | (fp8 ? EP_DISPATCH_FP8 : 0u);
    EP_OK_(ep_dispatch(h, flags, d_x, d_w, d_rx, fp8 ? d_sc : nullptr, d_rw, d_meta, nullptr));
    HIP_OK(hipDeviceSynchronize());
    std::vector<uint8_t> rx(R * row_bytes), orx(R * row_bytes);
    std::vector<float> sc(R * (H / 128)), osc(R * (H / 128)), rw(R), orw(R);
    std::vector<int32_t> meta(R * 2), ometa(R * 2);
    HIP_OK(hipMemcpy(rx.data(), d_rx, rx.size(), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sc.data(), d_sc, sc.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(rw.data(), d_rw, R * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(meta.data(), d_meta, R * 8, hipMemcpyDeviceToHost));
    if (oracle_dispatch(P, S, E, K, H, A, fp8, 1, topk.data(), dst_slot.data(), ne_tot.data(), eoff.data(),
                        wbase.data(), x.data(), w.data(), 0, R, orx.data(), osc.data(), orw.data(),
                        ometa.data()) != ORACLE_OK)
      return 5;
    expect(rx == orx, fp8 ? "fp8 payload" : "bf16 payload");
    expect(std::memcmp(rw.data(), orw.data(), R * 4) == 0, "recv_weights");
    expect(meta == ometa, "recv_src_meta");
    if (fp8) expect(std::memcmp(sc.data(), osc.data(), sc.size() * 4) == 0, "fp8 scales");

    // cached dispatch of the same x reproduces the payload
    HIP_OK(hipMemset(d_rx, 0x5A, R * row_bytes));
    EP_OK_(ep_dispatch_cached(h, flags, d_x, d_rx, fp8 ? d_sc : nullptr, nullptr));
    HIP_OK(hipDeviceSynchronize());
    std::vector<uint8_t> crx(R * row_bytes);
    HIP_OK(hipMemcpy(crx.data(), d_rx, crx.size(), hipMemcpyDeviceToHost));
    expect(crx == orx, "cached payload");

    if (!fp8) {  // combine of the dispatched rows (identity experts)
      uint16_t* d_out;
      HIP_OK(hipMalloc((void**)&d_out, T * H * 2 + 16));
      EP_OK_(ep_combine(h, d_rx, d_w, nullptr, d_out, nullptr));
      HIP_OK(hipDeviceSynchronize());
      std::vector<uint16_t> out(T * H), oout(T * H);
      HIP_OK(hipMemcpy(out.data(), d_out, T * H * 2, hipMemcpyDeviceToHost));
      if (oracle_combine(P, S, E, K, H, topk.data(), dst_slot.data(), wbase.data(), (const uint16_t*)orx.data(),
                         w.data(), 0, T, oout.data()) != ORACLE_OK)
        return 5;
      expect(out == oout, "combine");
      HIP_OK(hipFree(d_out));
    }
    HIP_OK(hipFree(d_rx));
    HIP_OK(hipFree(d_sc));
    HIP_OK(hipFree(d_rw));
    HIP_OK(hipFree(d_meta));
  }

  // Output buffers sized by the host-only hint, as a caller allocating the
  // long-lived buffer once would: bf16 rows need max_rows * 2H bytes, fp8
  // rows max_rows * H plus H/32 scale bytes a row (fp32 per 128 channels or
  // UE8M0 per 32).
  ep_size_hint hb{}, h8{};
  EP_OK_(ep_buffer_size_hint(&cfg, EP_DISPATCH_ZERO_PADDING, &hb));
  EP_OK_(ep_buffer_size_hint(&cfg, EP_DISPATCH_FP8 | EP_DISPATCH_ZERO_PADDING, &h8));
  expect(hb.max_rows >= R && h8.max_rows == hb.max_rows, "size hint: max_rows bounds the layout");
  expect(hb.recv_x_bytes == hb.max_rows * 2 * H && h8.recv_x_bytes == h8.max_rows * H, "size hint: payload bytes");
  expect(h8.recv_scales_bytes == h8.max_rows * (H / 32) && hb.recv_scales_bytes == 0, "size hint: scale bytes");
  expect(hb.combine_out_bytes == T * H * 2 && hb.total_bytes % (2 << 20) == 0, "size hint: combine and total");
  void *d_hx = nullptr, *d_hsc = nullptr, *d_hrw = nullptr, *d_hmeta = nullptr;
  HIP_OK(hipMalloc(&d_hx, hb.recv_x_bytes));
  HIP_OK(hipMalloc(&d_hsc, h8.recv_scales_bytes));
  HIP_OK(hipMalloc(&d_hrw, hb.recv_weights_bytes));
  HIP_OK(hipMalloc(&d_hmeta, hb.recv_src_meta_bytes));
  {
    // fp8 with UE8M0 scales: one exponent byte per 32 channels, row-major
    std::vector<uint8_t> rx(R * H), orx(R * H), sc(R * (H / 32)), osc(R * (H / 32));
    HIP_OK(hipMemset(d_hsc, 0x33, h8.recv_scales_bytes));
    EP_OK_(ep_dispatch(h, EP_DISPATCH_SCALES_UE8M0 | EP_DISPATCH_ZERO_PADDING, d_x, d_w, d_hx, (float*)d_hsc,
                       (float*)d_hrw, (int32_t*)d_hmeta, nullptr));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(rx.data(), d_hx, rx.size(), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sc.data(), d_hsc, sc.size(), hipMemcpyDeviceToHost));
    if (oracle_dispatch_general(P, S, E, K, H, A, 1, 1, 2, 0, topk.data(), dst_slot.data(), ne_tot.data(),
                                eoff.data(), wbase.data(), x.data(), nullptr, nullptr, w.data(), 0, R, orx.data(),
                                (float*)osc.data(), nullptr, nullptr, nullptr) != ORACLE_OK)
      return 5;
    expect(rx == orx, "UE8M0 codes");
    expect(sc == osc, "UE8M0 exponent bytes");
  }
  {
    // the scratch-free dispatch, fp8 with column-major scales [H/128][R]
    const int nb = H / 128;
    std::vector<uint8_t> rx(R * H), orx(R * H);
    std::vector<float> sc(nb * R), osc(nb * R), rw(R), orw(R);
    std::vector<int32_t> meta(R * 2), ometa(R * 2);
    const uint32_t fl = EP_DISPATCH_FP8 | EP_DISPATCH_SCALES_COL_MAJOR | EP_DISPATCH_ZERO_PADDING;
    EP_OK_(ep_dispatch_noalloc(h, fl, d_x, d_w, d_hx, (float*)d_hsc, (float*)d_hrw, (int32_t*)d_hmeta, nullptr));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(rx.data(), d_hx, rx.size(), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sc.data(), d_hsc, sc.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(rw.data(), d_hrw, R * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(meta.data(), d_hmeta, R * 8, hipMemcpyDeviceToHost));
    if (oracle_dispatch_general(P, S, E, K, H, A, 1, 1, 1, 0, topk.data(), dst_slot.data(), ne_tot.data(),
                                eoff.data(), wbase.data(), x.data(), nullptr, nullptr, w.data(), 0, R, orx.data(),
                                osc.data(), orw.data(), ometa.data(), nullptr) != ORACLE_OK)
      return 5;
    expect(rx == orx, "no-alloc fp8 codes");
    expect(std::memcmp(sc.data(), osc.data(), sc.size() * 4) == 0, "no-alloc column-major scales");
    expect(std::memcmp(rw.data(), orw.data(), R * 4) == 0 && meta == ometa, "no-alloc weights and meta");
  }
  ep_handle_free(h);
  HIP_OK(hipFree(d_hx));
  HIP_OK(hipFree(d_hsc));
  HIP_OK(hipFree(d_hrw));
  HIP_OK(hipFree(d_hmeta));

  {
    // fixed-length windows: W rows per window, no read-back, zero tails
    int64_t W = 0;
    for (int r = 0; r < P; ++r) W = std::max<int64_t>(W, nexp[r]);
    W += 3;
    ep_config cf = cfg;
    cf.num_worst_rows = (int32_t)W;
    ep_size_hint hf{};
    EP_OK_(ep_buffer_size_hint(&cf, EP_DISPATCH_ZERO_PADDING, &hf));
    ep_handle* hx = nullptr;
    int64_t rows_f = -1;
    EP_OK_(ep_get_layout(&cf, d_topk, nullptr, &hx, &rows_f));
    expect(rows_f == P * W && hf.max_rows == P * W, "fixed windows: P * W rows");
    void *d_fx, *d_frw, *d_fmeta;
    uint16_t* d_fout;
    HIP_OK(hipMalloc(&d_fx, hf.recv_x_bytes));
    HIP_OK(hipMalloc(&d_frw, hf.recv_weights_bytes));
    HIP_OK(hipMalloc(&d_fmeta, hf.recv_src_meta_bytes));
    HIP_OK(hipMalloc((void**)&d_fout, hf.combine_out_bytes));
    HIP_OK(hipMemset(d_fx, 0x5A, hf.recv_x_bytes));
    EP_OK_(ep_dispatch(hx, EP_DISPATCH_ZERO_PADDING, d_x, d_w, d_fx, nullptr, (float*)d_frw, (int32_t*)d_fmeta,
                       nullptr));
    EP_OK_(ep_combine(hx, d_fx, d_w, nullptr, d_fout, nullptr));
    HIP_OK(hipDeviceSynchronize());
    uint32_t st_flags = 99;
    int64_t dropped = -1;
    EP_OK_(ep_handle_status(hx, &st_flags, &dropped));
    expect(st_flags == 0 && dropped == 0, "fixed windows: status");
    const int64_t RF = P * W;
    std::vector<uint16_t> fx(RF * H), ofx(RF * H), fout(T * H), ofout(T * H);
    std::vector<float> frw(RF), ofrw(RF);
    std::vector<int32_t> fmeta(RF * 2), ofmeta(RF * 2);
    HIP_OK(hipMemcpy(fx.data(), d_fx, RF * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(frw.data(), d_frw, RF * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(fmeta.data(), d_fmeta, RF * 8, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(fout.data(), d_fout, T * H * 2, hipMemcpyDeviceToHost));
    int64_t odropped = -1;
    if (oracle_dispatch_general(P, S, E, K, H, A, 0, 1, 0, W, topk.data(), dst_slot.data(), ne_tot.data(),
                                eoff.data(), nullptr, x.data(), nullptr, nullptr, w.data(), 0, RF, ofx.data(),
                                nullptr, ofrw.data(), ofmeta.data(), &odropped) != ORACLE_OK ||
        oracle_combine_general(P, S, E, K, H, W, topk.data(), dst_slot.data(), nullptr, ofx.data(), w.data(),
                               nullptr, 0, T, ofout.data()) != ORACLE_OK)
      return 5;
    expect(odropped == 0, "fixed windows: the oracle drops nothing");
    expect(fx == ofx, "fixed windows: payload and zero tails");
    expect(std::memcmp(frw.data(), ofrw.data(), RF * 4) == 0 && fmeta == ofmeta, "fixed windows: weights and meta");
    expect(fout == ofout, "fixed windows: combine");
    ep_handle_free(hx);
    HIP_OK(hipFree(d_fx));
    HIP_OK(hipFree(d_frw));
    HIP_OK(hipFree(d_fmeta));
    HIP_OK(hipFree(d_fout));
  }
  HIP_OK(hipFree(d_topk));
  HIP_OK(hipFree(d_x));
  HIP_OK(hipFree(d_w));
  if (failures) {
    std::printf("c_abi roundtrip: %d mismatches\n", failures);
    return 1;
  }
  std::printf("c_abi roundtrip: ok (P=%d S=%d E=%d K=%d H=%d A=%d, %lld rows)\n", P, S, E, K, H, A, (long long)R);
  return 0;
}

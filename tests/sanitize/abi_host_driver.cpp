// Host-side checks of the library's C ABI, built together with the library's
// own API source (csrc/mla_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU:
//  * every validation clause of every entry point, with placeholder pointer
//    values that are never dereferenced (a rejected call queues nothing);
//  * zero-token calls, which are no-ops;
//  * the host-only planners (split-KV launch size, workspace size) over a
//    sweep of extreme argument values;
//  * status strings of every status value, valid or not;
//  * the thread-local error message, set by different rejections in
//    several threads at once.
// The kernel launchers are replaced by stubs that abort: a CPU call that
// reached one would be a validation hole.  Prints "ok" and exits 0 when
// every check passes.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <string>
#include <thread>
#include <vector>

#include "mla.h"
#include "mla_internal.h"

namespace mla {
[[noreturn]] static void reached(const char *what) {
  std::fprintf(stderr, "FAIL: %s reached on the host-only build\n", what);
  std::abort();
}
hipError_t launch_sparse_fwd(const FwdArgs &, hipStream_t) { reached("launch_sparse_fwd"); }
hipError_t launch_cache_insert(const InsertArgs &, hipStream_t) { reached("launch_cache_insert"); }
hipError_t launch_decode_epilogue(const DecodeEpilogueArgs &, hipStream_t) { reached("launch_decode_epilogue"); }
hipError_t launch_prefill_epilogue(const PrefillEpilogueArgs &, hipStream_t) { reached("launch_prefill_epilogue"); }
hipError_t launch_gather_upconvert(const GatherArgs &, hipStream_t) { reached("launch_gather_upconvert"); }
hipError_t launch_v_up_proj(const VUpProjArgs &, int, hipStream_t) { reached("launch_v_up_proj"); }
hipError_t launch_prepare_w_uv(const uint16_t *, uint16_t *, int32_t, hipStream_t) { reached("launch_prepare_w_uv"); }
}  // namespace mla

namespace {

constexpr mla_status_t OK = MLA_OK, INVALID = MLA_ERR_INVALID_ARGUMENT, UNSUP = MLA_ERR_UNSUPPORTED;
// A 256-byte aligned placeholder address, and offsets from it.
char *const P = reinterpret_cast<char *>(static_cast<uintptr_t>(0x100000));

int failures = 0;

void expect(const std::string &what, mla_status_t got, mla_status_t want) {
  const char *msg = mla_last_error();
  const bool msg_ok = want == OK || (msg != nullptr && msg[0] != '\0');
  if (got != want || !msg_ok) {
    std::fprintf(stderr, "FAIL %s: status %d, want %d (%s)\n", what.c_str(), (int)got, (int)want,
                 msg ? msg : "(null message)");
    ++failures;
  }
}

template <typename Args>
void run_cases(const char *name, const Args &base, const std::function<mla_status_t(const Args &)> &call,
               const std::vector<std::pair<std::function<void(Args &)>, mla_status_t>> &cases) {
  for (size_t i = 0; i < cases.size(); ++i) {
    Args a = base;
    cases[i].first(a);
    expect(std::string(name) + " case " + std::to_string(i), call(a), cases[i].second);
  }
}

struct Fwd {
  const void *q = P;
  int64_t T = 4;
  int32_t H = 16;
  int64_t qst = 16 * 576, qsh = 576;
  const void *kv = P;
  int64_t n = 100, pitch = 656;
  const void *indptr = P, *indices = P;
  int64_t nnz = 10;
  float scale = 1.0f;
  uint32_t flags = MLA_FLAG_RETURN_LSE;
  void *out = P;
  int64_t ost = 16 * 512, osh = 512;
  float *lse = reinterpret_cast<float *>(P);
  // second segment and sink (the _ex entry point)
  const float *sink = nullptr;
  const void *erec = P;
  int64_t en = 50, epitch = 656;
  const void *eptr = P, *eidx = P;
  int64_t ennz = 10;
  // the up-projection of mla_sparse_fwd_v_up_proj
  const void *vw = P;
  const void *vgate = nullptr;
  int64_t vgst = 0;
  void *vout = P;
  int64_t vst = 16 * 128, vsh = 128;
};

mla_status_t call_fwd(const Fwd &a) {
  return mla_sparse_fwd(a.q, a.T, a.H, a.qst, a.qsh, a.kv, a.n, a.pitch, a.indptr, a.indices, a.nnz, a.scale,
                        a.flags, a.out, a.ost, a.osh, a.lse, nullptr, 0, nullptr);
}
mla_status_t call_noalloc(const Fwd &a) {
  return mla_sparse_fwd_noalloc(a.q, a.T, a.H, a.qst, a.qsh, a.kv, a.n, a.pitch, a.indptr, a.indices, a.nnz, a.scale,
                                a.flags, a.out, a.ost, a.osh, a.lse, nullptr);
}
mla_status_t call_fwd_vp(const Fwd &a) {
  return mla_sparse_fwd_v_up_proj(a.q, a.T, a.H, a.qst, a.qsh, a.kv, a.n, a.pitch, a.indptr, a.indices, a.nnz, a.scale,
                                  a.flags, a.out, a.ost, a.osh, a.lse, a.vw, a.vgate, a.vgst, a.vout, a.vst, a.vsh,
                                  nullptr, 0, nullptr);
}
mla_status_t call_fwd_ex(const Fwd &a) {
  return mla_sparse_fwd_ex(a.q, a.T, a.H, a.qst, a.qsh, a.kv, a.n, a.pitch, a.indptr, a.indices, a.nnz, a.sink,
                           a.erec, a.en, a.epitch, a.eptr, a.eidx, a.ennz, a.scale, a.flags, a.out, a.ost, a.osh,
                           a.lse, nullptr, 0, nullptr);
}

std::vector<std::pair<std::function<void(Fwd &)>, mla_status_t>> fwd_cases() {
  return {
      {[](Fwd &a) { a.H = 0; }, UNSUP},
      {[](Fwd &a) { a.H = 17; }, UNSUP},
      {[](Fwd &a) { a.T = -1; }, INVALID},
      {[](Fwd &a) { a.qst = 16 * 576 + 1; }, UNSUP},
      {[](Fwd &a) { a.qsh = 577; }, UNSUP},
      {[](Fwd &a) { a.ost = 8191; }, UNSUP},
      {[](Fwd &a) { a.osh = -2; }, INVALID},
      {[](Fwd &a) { a.q = P + 2; }, UNSUP},
      {[](Fwd &a) { a.out = P + 2; }, UNSUP},
      {[](Fwd &a) { a.kv = P + 8; }, UNSUP},
      {[](Fwd &a) { a.pitch = 672; }, UNSUP},
      {[](Fwd &a) { a.pitch = 64 * 672; }, UNSUP},
      {[](Fwd &a) { a.n = -1; }, INVALID},
      {[](Fwd &a) { a.nnz = int64_t(1) << 29; }, UNSUP},
      {[](Fwd &a) { a.nnz = -3; }, INVALID},
      {[](Fwd &a) { a.nnz = INT64_MAX; }, UNSUP},
      {[](Fwd &a) { a.flags = 1u << 7; }, INVALID},
      {[](Fwd &a) { a.lse = nullptr; }, INVALID},
      {[](Fwd &a) { a.lse = reinterpret_cast<float *>(P + 1); }, INVALID},
      {[](Fwd &a) { a.indptr = P + 2; }, INVALID},
      {[](Fwd &a) { a.flags |= MLA_FLAG_INDEX_I64; a.indices = P + 4; }, INVALID},
      {[](Fwd &a) { a.q = nullptr; }, INVALID},
      {[](Fwd &a) { a.out = nullptr; }, INVALID},
      {[](Fwd &a) { a.indptr = nullptr; }, INVALID},
      {[](Fwd &a) { a.indices = nullptr; }, INVALID},
      {[](Fwd &a) { a.T = 513; a.flags |= MLA_FLAG_CHUNK_TILES(4); }, UNSUP},
      {[](Fwd &a) { a.T = INT64_MAX; }, UNSUP},
      {[](Fwd &a) { a.qst = INT64_MAX - 1; }, INVALID},
      {[](Fwd &a) { a.osh = int64_t(1) << 60; }, INVALID},
      {[](Fwd &a) { a.T = 0; a.q = nullptr; a.out = nullptr; a.indptr = nullptr; a.indices = nullptr;
                    a.lse = nullptr; }, OK},
  };
}

struct Ins {
  const void *kv_c = P;
  int64_t kst = 512;
  const void *k_pe = P;
  int64_t pst = 64;
  const int64_t *slots = reinterpret_cast<const int64_t *>(P);
  int64_t T = 8;
  void *kv = P;
  int64_t n = 100, pitch = 656;
};

struct Epi {
  const void *ql = P;
  int64_t qlt = 16 * 512, qlh = 512;
  const void *qp = P;
  int64_t qpt = 16 * 64, qph = 64;
  const void *kv = P;
  int64_t kvt = 512;
  const void *kp = P;
  int64_t kpt = 64;
  const int64_t *slots = reinterpret_cast<const int64_t *>(P);
  int64_t T = 8;
  int32_t H = 16;
  const int64_t *pos = nullptr;
  const float *cs = nullptr;
  int64_t maxpos = 0;
  void *mq = P;
  int64_t mqt = 16 * 576, mqh = 576;
  void *rec = P;
  int64_t n = 100, pitch = 656;
};

struct Pre {
  void *q = P;
  int64_t qst = 16 * 192, qsh = 192;
  int32_t nope = 128;
  const void *kn = P;
  int64_t knt = 16 * 128, knh = 128;
  const void *kv = P;
  int64_t kvt = 512;
  const void *kp = P;
  int64_t kpt = 64;
  const int64_t *slots = reinterpret_cast<const int64_t *>(P);
  int64_t T = 8;
  int32_t H = 16;
  const int64_t *pos = nullptr;
  const float *cs = nullptr;
  int64_t maxpos = 0;
  void *ko = P;
  int64_t kot = 16 * 192, koh = 192;
  void *rec = P;
  int64_t n = 100, pitch = 656;
};

struct Gat {
  const void *rec = P;
  int64_t n = 1024, pitch = 656, bs = 64;
  const int32_t *bt = reinterpret_cast<const int32_t *>(P);
  int64_t bts = 16, btw = 16;
  const int32_t *cu = reinterpret_cast<const int32_t *>(P);
  const int32_t *starts = nullptr;
  int32_t B = 8;
  int64_t T = 100;
  void *dst = P;
  int64_t dsts = 576;
};

struct Vp {
  const void *lat = P;
  int64_t lst = 16 * 512, lsh = 512;
  const void *w = P;
  const void *gate = nullptr;
  int64_t gst = 0, T = 64;
  int32_t H = 16;
  void *out = P;
  int64_t ost = 16 * 128, osh = 128;
};

void check_planners() {
  const int64_t tokens[] = {-1, 0, 1, 7, 8, 63, 64, 511, 512, 513, 4096, INT32_MAX, INT64_MAX / 2, INT64_MAX};
  const int64_t nnzs[] = {-1, 0, 1, 100, 294271, (int64_t(1) << 29) - 1, int64_t(1) << 29, INT64_MAX};
  const int32_t cus[] = {-1, 0, 1, 256, INT32_MAX};
  const uint32_t flags[] = {0u, MLA_FLAG_CHUNK_TILES(1), MLA_FLAG_CHUNK_TILES(7), MLA_FLAG_CHUNK_MASK, 1u << 5,
                            MLA_FLAG_RETURN_LSE | MLA_FLAG_CHUNK_TILES(64)};
  int64_t sink = 0;
  for (int64_t t : tokens)
    for (int64_t z : nnzs)
      for (int32_t c : cus)
        for (uint32_t f : flags) sink += mla_sparse_fwd_split_workgroups(t, z, c, f);
  // forced chunks need no device; H beyond 16 and negative sizes are refused
  const int32_t heads[] = {-1, 0, 1, 16, 17, INT32_MAX};
  size_t total = 0;
  for (int64_t t : tokens)
    for (int64_t z : nnzs)
      for (int32_t h : heads)
        for (uint32_t f : {MLA_FLAG_CHUNK_TILES(1), MLA_FLAG_CHUNK_TILES(4), MLA_FLAG_CHUNK_MASK})
          total += mla_sparse_fwd_workspace_size(t, h, z, f, 0);
  // values the ABI tests also pin
  if (mla_sparse_fwd_split_workgroups(8, 8 * 131072, 256, 0) != 512) { std::fprintf(stderr, "FAIL plan 1\n"); ++failures; }
  if (mla_sparse_fwd_split_workgroups(4096, int64_t(4096) * 2048, 256, 0) != 0) { std::fprintf(stderr, "FAIL plan 2\n"); ++failures; }
  if (mla_sparse_fwd_split_workgroups(-1, 0, 256, 0) != -1) { std::fprintf(stderr, "FAIL plan 3\n"); ++failures; }
  if (mla_sparse_fwd_workspace_size(8, 17, 1000, MLA_FLAG_CHUNK_TILES(4), 0) != (size_t)-1) {
    std::fprintf(stderr, "FAIL workspace 17 heads\n");
    ++failures;
  }
  std::printf("planners swept (%lld, %zu)\n", (long long)sink, total);
}

void check_threads() {
  // each thread makes its own rejected call and must read back its own message
  std::vector<std::thread> ts;
  std::vector<int> bad(8, 0);
  for (int i = 0; i < 8; ++i) {
    ts.emplace_back([i, &bad] {
      for (int k = 0; k < 200; ++k) {
        Fwd a;
        a.H = 17 + i;  // each thread's own head count appears in its message
        const mla_status_t st = call_fwd(a);
        const std::string want = std::to_string(17 + i);
        if (st != UNSUP || std::strstr(mla_last_error(), want.c_str()) == nullptr) bad[i] = 1;
      }
    });
  }
  for (auto &t : ts) t.join();
  for (int i = 0; i < 8; ++i)
    if (bad[i]) {
      std::fprintf(stderr, "FAIL thread %d read another thread's message\n", i);
      ++failures;
    }
}

}  // namespace

int main() {
  if (mla_abi_version() != MLA_ABI_VERSION) {
    std::fprintf(stderr, "FAIL abi version\n");
    return 1;
  }
  for (int s = -3; s < 12; ++s) {
    const char *str = mla_status_string(static_cast<mla_status_t>(s));
    if (str == nullptr || str[0] == '\0') {
      std::fprintf(stderr, "FAIL status string %d\n", s);
      ++failures;
    }
  }

  run_cases<Fwd>("mla_sparse_fwd", Fwd{}, call_fwd, fwd_cases());
  run_cases<Fwd>("mla_sparse_fwd_noalloc", Fwd{}, call_noalloc, fwd_cases());
  {
    // the forward's cases through the forward + projection entry point (its
    // own conditions hold with these placeholders), then the projection's
    auto vp_cases = fwd_cases();
    vp_cases.insert(vp_cases.end(), {
        {[](Fwd &a) { a.out = P + 8; }, UNSUP},
        {[](Fwd &a) { a.ost = 16 * 512 + 2; }, UNSUP},
        {[](Fwd &a) { a.vw = P + 8; }, UNSUP},
        {[](Fwd &a) { a.vout = P + 2; }, UNSUP},
        {[](Fwd &a) { a.vsh = 129; }, UNSUP},
        {[](Fwd &a) { a.vgate = P; a.vgst = 2049; }, UNSUP},
        {[](Fwd &a) { a.vst = int64_t(1) << 61; }, INVALID},
        {[](Fwd &a) { a.vw = nullptr; }, INVALID},
        {[](Fwd &a) { a.vout = nullptr; }, INVALID},
    });
    // the forward's out-alignment case (P + 2) is refused for 16-byte alignment
    // first, so its status here is the same UNSUPPORTED
    run_cases<Fwd>("mla_sparse_fwd_v_up_proj", Fwd{}, call_fwd_vp, vp_cases);
  }
  auto ex_cases = fwd_cases();
  ex_cases.insert(ex_cases.end(), {
      {[](Fwd &a) { a.epitch = 672; }, UNSUP},
      {[](Fwd &a) { a.en = -1; }, INVALID},
      {[](Fwd &a) { a.en = (int64_t(1) << 31) - 2; }, UNSUP},
      {[](Fwd &a) { a.ennz = (int64_t(1) << 29) - 10; }, UNSUP},
      {[](Fwd &a) { a.ennz = INT64_MAX; }, UNSUP},
      {[](Fwd &a) { a.erec = P + 8; }, UNSUP},
      {[](Fwd &a) { a.eptr = P + 2; }, INVALID},
      {[](Fwd &a) { a.eidx = nullptr; }, INVALID},
      {[](Fwd &a) { a.sink = reinterpret_cast<const float *>(P + 2); }, INVALID},
  });
  run_cases<Fwd>("mla_sparse_fwd_ex", Fwd{}, call_fwd_ex, ex_cases);

  run_cases<Ins>("mla_cache_insert", Ins{},
                 [](const Ins &a) { return mla_cache_insert(a.kv_c, a.kst, a.k_pe, a.pst, a.slots, a.T, a.kv, a.n, a.pitch, nullptr); },
                 {
                     {[](Ins &a) { a.T = -1; }, INVALID},
                     {[](Ins &a) { a.kst = 511; }, UNSUP},
                     {[](Ins &a) { a.pst = -64; }, INVALID},
                     {[](Ins &a) { a.pitch = 660; }, UNSUP},
                     {[](Ins &a) { a.kv = P + 4; }, UNSUP},
                     {[](Ins &a) { a.kv_c = P + 2; }, UNSUP},
                     {[](Ins &a) { a.k_pe = P + 1; }, UNSUP},
                     {[](Ins &a) { a.slots = reinterpret_cast<const int64_t *>(P + 4); }, INVALID},
                     {[](Ins &a) { a.n = -5; }, INVALID},
                     {[](Ins &a) { a.kv_c = nullptr; }, INVALID},
                     {[](Ins &a) { a.slots = nullptr; }, INVALID},
                     {[](Ins &a) { a.T = INT64_MAX; }, INVALID},  // its kv_c view spans past 2^62
                     {[](Ins &a) { a.kst = int64_t(1) << 61; }, INVALID},
                     {[](Ins &a) { a.n = INT64_MAX; }, UNSUP},
                     {[](Ins &a) { a.T = 0; a.kv_c = nullptr; a.k_pe = nullptr; a.slots = nullptr; }, OK},
                 });

  run_cases<Epi>("mla_decode_q_concat_insert", Epi{},
                 [](const Epi &a) {
                   return mla_decode_q_concat_insert(a.ql, a.qlt, a.qlh, a.qp, a.qpt, a.qph, a.kv, a.kvt, a.kp, a.kpt,
                                                     a.slots, a.T, a.H, a.pos, a.cs, a.maxpos, a.mq, a.mqt, a.mqh,
                                                     a.rec, a.n, a.pitch, nullptr);
                 },
                 {
                     {[](Epi &a) { a.H = 0; }, UNSUP},
                     {[](Epi &a) { a.H = 1025; }, UNSUP},
                     {[](Epi &a) { a.T = -1; }, INVALID},
                     {[](Epi &a) { a.qlh = 511; }, UNSUP},
                     {[](Epi &a) { a.qpt = -64; }, INVALID},
                     {[](Epi &a) { a.mqh = 577; }, UNSUP},
                     {[](Epi &a) { a.ql = P + 2; }, UNSUP},
                     {[](Epi &a) { a.mq = P + 2; }, UNSUP},
                     {[](Epi &a) { a.pitch = 672; }, UNSUP},
                     {[](Epi &a) { a.rec = P + 8; }, UNSUP},
                     {[](Epi &a) { a.n = -1; }, INVALID},
                     {[](Epi &a) { a.slots = reinterpret_cast<const int64_t *>(P + 4); }, INVALID},
                     {[](Epi &a) { a.pos = reinterpret_cast<const int64_t *>(P); }, INVALID},
                     {[](Epi &a) { a.cs = reinterpret_cast<const float *>(P); a.maxpos = 16; }, INVALID},
                     {[](Epi &a) { a.pos = reinterpret_cast<const int64_t *>(P); a.cs = reinterpret_cast<const float *>(P); }, INVALID},
                     {[](Epi &a) { a.pos = reinterpret_cast<const int64_t *>(P + 4); a.cs = reinterpret_cast<const float *>(P); a.maxpos = 16; }, INVALID},
                     {[](Epi &a) { a.ql = nullptr; }, INVALID},
                     {[](Epi &a) { a.mq = nullptr; }, INVALID},
                     {[](Epi &a) { a.mqt = int64_t(1) << 60; }, INVALID},
                     {[](Epi &a) { a.n = int64_t(1) << 41; }, UNSUP},
                     {[](Epi &a) { a.pos = reinterpret_cast<const int64_t *>(P); a.cs = reinterpret_cast<const float *>(P);
                                   a.maxpos = INT64_MAX; }, UNSUP},
                     {[](Epi &a) { a.T = 0; a.ql = nullptr; a.qp = nullptr; a.kv = nullptr; a.kp = nullptr;
                                   a.slots = nullptr; a.mq = nullptr; }, OK},
                 });

  run_cases<Pre>("mla_prefill_key_concat_insert", Pre{},
                 [](const Pre &a) {
                   return mla_prefill_key_concat_insert(a.q, a.qst, a.qsh, a.nope, a.kn, a.knt, a.knh, a.kv, a.kvt,
                                                        a.kp, a.kpt, a.slots, a.T, a.H, a.pos, a.cs, a.maxpos, a.ko,
                                                        a.kot, a.koh, a.rec, a.n, a.pitch, nullptr);
                 },
                 {
                     {[](Pre &a) { a.nope = 0; }, UNSUP},
                     {[](Pre &a) { a.nope = 100; }, UNSUP},
                     {[](Pre &a) { a.nope = 2048; }, UNSUP},
                     {[](Pre &a) { a.H = 0; }, UNSUP},
                     {[](Pre &a) { a.knh = 129; }, UNSUP},
                     {[](Pre &a) { a.qst = -2; }, INVALID},
                     {[](Pre &a) { a.ko = P + 2; }, UNSUP},
                     {[](Pre &a) { a.pos = reinterpret_cast<const int64_t *>(P); }, INVALID},
                     {[](Pre &a) { a.pos = reinterpret_cast<const int64_t *>(P); a.cs = reinterpret_cast<const float *>(P);
                                   a.maxpos = 16; a.q = nullptr; }, INVALID},
                     {[](Pre &a) { a.pitch = 672; }, UNSUP},
                     {[](Pre &a) { a.kn = nullptr; }, INVALID},
                     {[](Pre &a) { a.koh = int64_t(1) << 60; }, INVALID},
                     {[](Pre &a) { a.n = int64_t(1) << 41; }, UNSUP},
                     {[](Pre &a) { a.T = 0; a.q = nullptr; a.kn = nullptr; a.kv = nullptr; a.kp = nullptr;
                                   a.slots = nullptr; a.ko = nullptr; }, OK},
                 });

  run_cases<Gat>("mla_gather_upconvert", Gat{},
                 [](const Gat &a) {
                   return mla_gather_upconvert(a.rec, a.n, a.pitch, a.bs, a.bt, a.bts, a.btw, a.cu, a.starts, a.B,
                                               a.T, a.dst, a.dsts, nullptr);
                 },
                 {
                     {[](Gat &a) { a.T = -1; }, INVALID},
                     {[](Gat &a) { a.n = -1; }, INVALID},
                     {[](Gat &a) { a.B = -1; }, INVALID},
                     {[](Gat &a) { a.bs = 0; }, INVALID},
                     {[](Gat &a) { a.pitch = 660; }, UNSUP},
                     {[](Gat &a) { a.rec = P + 8; }, UNSUP},
                     {[](Gat &a) { a.dst = P + 8; }, UNSUP},
                     {[](Gat &a) { a.dsts = 580; }, UNSUP},
                     {[](Gat &a) { a.dsts = 512; }, UNSUP},
                     {[](Gat &a) { a.bt = reinterpret_cast<const int32_t *>(P + 2); }, INVALID},
                     {[](Gat &a) { a.cu = nullptr; }, INVALID},
                     {[](Gat &a) { a.bt = nullptr; }, INVALID},
                     {[](Gat &a) { a.dst = nullptr; }, INVALID},
                     {[](Gat &a) { a.dsts = int64_t(1) << 61; }, INVALID},
                     {[](Gat &a) { a.bts = int64_t(1) << 61; }, INVALID},
                     {[](Gat &a) { a.bs = int64_t(1) << 40; }, UNSUP},
                     {[](Gat &a) { a.n = int64_t(1) << 41; }, UNSUP},
                     {[](Gat &a) { a.T = 0; a.dst = nullptr; a.cu = nullptr; a.bt = nullptr; }, OK},
                 });

  auto vcall = [](const Vp &a) {
    return mla_v_up_proj(a.lat, a.lst, a.lsh, a.w, a.gate, a.gst, a.T, a.H, a.out, a.ost, a.osh, nullptr);
  };
  auto vpcall = [](const Vp &a) {
    return mla_v_up_proj_prepared(a.lat, a.lst, a.lsh, a.w, a.gate, a.gst, a.T, a.H, a.out, a.ost, a.osh, nullptr);
  };
  run_cases<Vp>("mla_v_up_proj", Vp{}, vcall,
                {
                    {[](Vp &a) { a.T = -1; }, INVALID},
                    {[](Vp &a) { a.H = 0; }, UNSUP},
                    {[](Vp &a) { a.H = 1025; }, UNSUP},
                    {[](Vp &a) { a.lst = -8; }, INVALID},
                    {[](Vp &a) { a.lsh = 516; }, UNSUP},
                    {[](Vp &a) { a.lat = P + 8; }, UNSUP},
                    {[](Vp &a) { a.out = P + 2; }, UNSUP},
                    {[](Vp &a) { a.osh = 129; }, UNSUP},
                    {[](Vp &a) { a.gate = P + 2; a.gst = 2048; }, UNSUP},
                    {[](Vp &a) { a.gate = P; a.gst = 2049; }, UNSUP},
                    {[](Vp &a) { a.lat = nullptr; }, INVALID},
                    {[](Vp &a) { a.w = nullptr; }, INVALID},
                    {[](Vp &a) { a.lst = int64_t(1) << 61; }, INVALID},
                    {[](Vp &a) { a.gate = P; a.gst = int64_t(1) << 61; }, INVALID},
                    {[](Vp &a) { a.T = 0; a.lat = nullptr; a.w = nullptr; a.out = nullptr; }, OK},
                });
  run_cases<Vp>("mla_v_up_proj_prepared", Vp{}, vpcall,
                {
                    {[](Vp &a) { a.H = 0; }, UNSUP},
                    {[](Vp &a) { a.w = P + 2; }, UNSUP},
                    {[](Vp &a) { a.w = nullptr; }, INVALID},
                    {[](Vp &a) { a.lat = P + 8; }, UNSUP},
                });
  expect("prepare_weights H=0", mla_v_up_proj_prepare_weights(P, 0, P + (1 << 24), nullptr), UNSUP);
  expect("prepare_weights H=1025", mla_v_up_proj_prepare_weights(P, 1025, P + (1 << 30), nullptr), UNSUP);
  expect("prepare_weights null in", mla_v_up_proj_prepare_weights(nullptr, 16, P, nullptr), INVALID);
  expect("prepare_weights null out", mla_v_up_proj_prepare_weights(P, 16, nullptr, nullptr), INVALID);
  expect("prepare_weights misaligned", mla_v_up_proj_prepare_weights(P, 16, P + 8 + (1 << 24), nullptr), UNSUP);
  expect("prepare_weights overlap", mla_v_up_proj_prepare_weights(P, 16, P + 4096, nullptr), INVALID);

  // no device on this host: a reserve names its device and fails cleanly
  const mla_status_t rs = mla_workspace_reserve(-1, 1 << 20);
  if (rs == OK || mla_last_error()[0] == '\0') {
    std::fprintf(stderr, "FAIL workspace_reserve(-1)\n");
    ++failures;
  }

  check_planners();
  check_threads();

  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::puts("ok");
  return 0;
}

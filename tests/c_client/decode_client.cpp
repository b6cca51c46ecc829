// A C-ABI client of the paged decode library, as a non-Python engine would
// drive it: raw HIP allocations, the header's declarations, status codes.
//
// Usage: decode_client <dir>
//   reads  <dir>/meta.txt      "batch num_pages max_blocks max_seq_len pages_per_split
//                               [bits [launch [heads_together]]]"
//                              (bits: 16 BF16 pages, the default; 8 INT8; 4 INT4;
//                               launch: 0 the split grid, the default; 1 the balanced
//                               launch of pa_decode_balanced.h over a plan built here
//                               from the host lengths, heads_together 8 by default;
//                               2 the allocation-free step, BF16 pages)
//          <dir>/q.bin         BF16 bits [batch][32][64]
//          <dir>/k_new.bin     BF16 bits [batch][8][64]   (v_new.bin likewise)
//          <dir>/k_pool.bin    BF16 bits [num_pages][16][8][64] (v_pool.bin likewise);
//                              quantised pages: the code pools (INT8 [num_pages][8][16][64]
//                              bytes, INT4 [num_pages][8][16][32]) and
//          <dir>/scales.bin    float32 [num_pages][8][2][16]
//          <dir>/bt.bin        int32 [batch][max_blocks]
//          <dir>/lens.bin      int32 [batch]
//   runs   pa_append_decode_attention (or _q8, _q4; FP32 out), pa_decode_balanced with
//          the fused append, or pa_append_decode_attention_noalloc, on the default stream
//   writes <dir>/out.bin       float32 [batch][32][64]
//          <dir>/k_pool_out.bin, v_pool_out.bin (and scales_out.bin): the pools after
//          the append
// Exits 0 on success, 1 on a library or HIP error (printed), 2 on bad input.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "pa_decode.h"
#include "pa_decode_balanced.h"
#include "pa_decode_q4.h"
#include "pa_decode_q8.h"

static bool read_file(const std::string& path, std::vector<char>& buf, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  buf.resize(bytes);
  const size_t got = std::fread(buf.data(), 1, bytes, f);
  std::fclose(f);
  return got == bytes;
}

static bool write_file(const std::string& path, const void* data, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const size_t put = std::fwrite(data, 1, bytes, f);
  std::fclose(f);
  return put == bytes;
}

#define HIP_OK(x)                                                                   \
  do {                                                                              \
    if ((x) != hipSuccess) {                                                        \
      std::fprintf(stderr, "HIP error at %s:%d\n", __FILE__, __LINE__);             \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  const std::string dir = argv[1];
  int batch = 0, num_pages = 0, max_blocks = 0, max_seq_len = 0, pps = 0, bits = 16;
  int launch = 0, heads_together = 8;
  {
    FILE* f = std::fopen((dir + "/meta.txt").c_str(), "r");
    if (!f || std::fscanf(f, "%d %d %d %d %d", &batch, &num_pages, &max_blocks, &max_seq_len,
                          &pps) != 5) return 2;
    if (std::fscanf(f, "%d", &bits) != 1) bits = 16;
    if (std::fscanf(f, "%d", &launch) != 1) launch = 0;
    if (std::fscanf(f, "%d", &heads_together) != 1) heads_together = 8;
    std::fclose(f);
  }
  if (batch < 1 || num_pages < 1 || max_blocks < 1) return 2;
  if (bits != 16 && bits != 8 && bits != 4) return 2;
  if (launch < 0 || launch > 2 || (launch == 2 && bits != 16)) return 2;
  const bool quant = bits != 16;
  const size_t q_b = (size_t)batch * 32 * 64 * 2, new_b = (size_t)batch * 8 * 64 * 2;
  // bytes per pool: 16 slots x 8 KV heads x 64 dims of `bits` each
  const size_t pool_b = (size_t)num_pages * 16 * 8 * 64 * bits / 8;
  const size_t scales_b = quant ? (size_t)num_pages * 8 * 2 * 16 * 4 : 0;
  const size_t bt_b = (size_t)batch * max_blocks * 4;
  const size_t lens_b = (size_t)batch * 4, out_b = (size_t)batch * 32 * 64 * 4;
  std::vector<char> q, kn, vn, kp, vp, sc, bt, lens;
  if (!read_file(dir + "/q.bin", q, q_b) || !read_file(dir + "/k_new.bin", kn, new_b) ||
      !read_file(dir + "/v_new.bin", vn, new_b) || !read_file(dir + "/k_pool.bin", kp, pool_b) ||
      !read_file(dir + "/v_pool.bin", vp, pool_b) || !read_file(dir + "/bt.bin", bt, bt_b) ||
      !read_file(dir + "/lens.bin", lens, lens_b) ||
      (quant && !read_file(dir + "/scales.bin", sc, scales_b)))
    return 2;

  pa_shape shape = {32, 8, 64, 16, num_pages, max_blocks};
  size_t ws_bytes = 0;
  int rc = pa_decode_workspace_bytes(&shape, batch, max_seq_len, pps, &ws_bytes);
  if (rc != PA_OK) { std::fprintf(stderr, "%s\n", pa_status_string(rc)); return 1; }

  void *dq, *dkn, *dvn, *dkp, *dvp, *dbt, *dlens, *dout, *dws = nullptr, *dsc = nullptr;
  HIP_OK(hipMalloc(&dq, q_b));
  HIP_OK(hipMalloc(&dkn, new_b));
  HIP_OK(hipMalloc(&dvn, new_b));
  HIP_OK(hipMalloc(&dkp, pool_b));
  HIP_OK(hipMalloc(&dvp, pool_b));
  HIP_OK(hipMalloc(&dbt, bt_b));
  HIP_OK(hipMalloc(&dlens, lens_b));
  HIP_OK(hipMalloc(&dout, out_b));
  if (ws_bytes) HIP_OK(hipMalloc(&dws, ws_bytes));
  HIP_OK(hipMemcpy(dq, q.data(), q_b, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dkn, kn.data(), new_b, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dvn, vn.data(), new_b, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dkp, kp.data(), pool_b, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dvp, vp.data(), pool_b, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dbt, bt.data(), bt_b, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, lens.data(), lens_b, hipMemcpyHostToDevice));
  if (quant) {
    HIP_OK(hipMalloc(&dsc, scales_b));
    HIP_OK(hipMemcpy(dsc, sc.data(), scales_b, hipMemcpyHostToDevice));
  }

  void* dplan = nullptr;
  if (launch == 1) {
    // the plan is built on the host from the lengths the device will hold
    int64_t words = 0;
    int32_t groups = 0;
    const int32_t* hl = (const int32_t*)lens.data();
    rc = pa_balance_plan(&shape, batch, hl, max_seq_len, 0, heads_together, nullptr, 0, &words,
                         &groups);
    if (rc != PA_OK) { std::fprintf(stderr, "%s\n", pa_status_string(rc)); return 1; }
    std::vector<int32_t> plan((size_t)words);
    rc = pa_balance_plan(&shape, batch, hl, max_seq_len, 0, heads_together, plan.data(), words,
                         &words, &groups);
    if (rc != PA_OK) { std::fprintf(stderr, "%s\n", pa_status_string(rc)); return 1; }
    HIP_OK(hipMalloc(&dplan, (size_t)words * 4));
    HIP_OK(hipMemcpy(dplan, plan.data(), (size_t)words * 4, hipMemcpyHostToDevice));
    rc = pa_decode_balanced(&shape, batch, dq, dkn, dvn, nullptr, dkp, dvp, dsc,
                            bits == 16 ? 0 : (bits == 8 ? 1 : 2), (const int32_t*)dbt,
                            (const int32_t*)dlens, max_seq_len, 0.125f, dout, PA_OUT_F32,
                            (const int32_t*)dplan, words, groups, nullptr);
  } else if (launch == 2)
    rc = pa_append_decode_attention_noalloc(&shape, batch, dq, dkn, dvn, dkp, dvp,
                                            (const int32_t*)dbt, (const int32_t*)dlens,
                                            max_seq_len, 0.125f, dout, PA_OUT_F32, pps, nullptr);
  else if (bits == 8)
    rc = pa_append_decode_attention_q8(&shape, batch, dq, dkn, dvn, dkp, dvp, dsc,
                                       (const int32_t*)dbt, (const int32_t*)dlens, max_seq_len,
                                       0.125f, dout, PA_OUT_F32, pps, dws, ws_bytes, nullptr);
  else if (bits == 4)
    rc = pa_append_decode_attention_q4(&shape, batch, dq, dkn, dvn, dkp, dvp, dsc,
                                       (const int32_t*)dbt, (const int32_t*)dlens, max_seq_len,
                                       0.125f, dout, PA_OUT_F32, pps, dws, ws_bytes, nullptr);
  else
    rc = pa_append_decode_attention(&shape, batch, dq, dkn, dvn, dkp, dvp, (const int32_t*)dbt,
                                    (const int32_t*)dlens, max_seq_len, 0.125f, dout, PA_OUT_F32,
                                    pps, dws, ws_bytes, nullptr);
  if (rc != PA_OK) { std::fprintf(stderr, "%s\n", pa_status_string(rc)); return 1; }
  // a host-checkable mistake is refused before any launch
  if (pa_append_decode_attention(&shape, batch, dq, dkn, dvn, dkp, dvp, (const int32_t*)dbt,
                                 (const int32_t*)dlens, max_seq_len, 0.125f, dout, 7, pps, dws,
                                 ws_bytes, nullptr) != PA_ERR_VALUE)
    return 1;
  HIP_OK(hipDeviceSynchronize());

  std::vector<char> out(out_b), kpo(pool_b), vpo(pool_b), sco(scales_b);
  HIP_OK(hipMemcpy(out.data(), dout, out_b, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(kpo.data(), dkp, pool_b, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(vpo.data(), dvp, pool_b, hipMemcpyDeviceToHost));
  if (quant) HIP_OK(hipMemcpy(sco.data(), dsc, scales_b, hipMemcpyDeviceToHost));
  for (void* p : {dq, dkn, dvn, dkp, dvp, dbt, dlens, dout}) HIP_OK(hipFree(p));
  if (dws) HIP_OK(hipFree(dws));
  if (dplan) HIP_OK(hipFree(dplan));
  if (dsc) HIP_OK(hipFree(dsc));
  if (!write_file(dir + "/out.bin", out.data(), out_b) ||
      !write_file(dir + "/k_pool_out.bin", kpo.data(), pool_b) ||
      !write_file(dir + "/v_pool_out.bin", vpo.data(), pool_b) ||
      (quant && !write_file(dir + "/scales_out.bin", sco.data(), scales_b)))
    return 2;
  std::printf("decode_client: batch %d, %d-bit pages, launch %d, abi %d, ok\n", batch, bits,
              launch, pa_abi_version());
  return 0;
}

// Test driver for the CPU MoE executor built on its own with the address and
// undefined-behaviour sanitizers (tests/test_cpu_moe_sanitized.py builds and
// runs it).  It reads one case from a binary file, runs oes_cpu_moe_run with
// each listed thread count and writes every y; it also walks the executor's
// argument errors.  Exit status: 0 when every call returned what it should.
//
// Input (little endian): int32 format, E, H, I, n, k, nthreads, threads[nthreads],
// nbanks, then per bank int64 bytes and the bytes; x bf16 [n, H]; ids int32
// [n, k]; slot_ids int32 [n, k]; w float [n, k].  Output: nthreads x y float [n, H].
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "oes.h"

static bool rd(FILE *f, void *p, size_t bytes) { return fread(p, 1, bytes, f) == bytes; }

#define CHECK(cond, ...)              \
  do {                                \
    if (!(cond)) {                    \
      fprintf(stderr, __VA_ARGS__);   \
      fprintf(stderr, "\n");          \
      return 1;                       \
    }                                 \
  } while (0)

int main(int argc, char **argv) {
  CHECK(argc == 3, "usage: %s in.bin out.bin", argv[0]);
  FILE *f = fopen(argv[1], "rb");
  CHECK(f, "cannot open %s", argv[1]);
  int32_t hd[7];
  CHECK(rd(f, hd, sizeof(hd)), "short header");
  const int32_t fmt = hd[0], E = hd[1], H = hd[2], I = hd[3], n = hd[4], k = hd[5], nth = hd[6];
  std::vector<int32_t> threads(nth);
  CHECK(rd(f, threads.data(), 4 * (size_t)nth), "short thread list");
  int32_t nb;
  CHECK(rd(f, &nb, 4), "short bank count");
  std::vector<std::vector<uint8_t>> banks(nb);
  for (auto &b : banks) {
    int64_t bytes;
    CHECK(rd(f, &bytes, 8), "short bank size");
    b.resize((size_t)bytes);
    CHECK(rd(f, b.data(), b.size()), "short bank");
  }
  std::vector<uint16_t> x((size_t)n * H);
  std::vector<int32_t> ids((size_t)n * k), slots((size_t)n * k);
  std::vector<float> w((size_t)n * k);
  CHECK(rd(f, x.data(), 2 * x.size()) && rd(f, ids.data(), 4 * ids.size()) && rd(f, slots.data(), 4 * slots.size()) &&
            rd(f, w.data(), 4 * w.size()),
        "short step inputs");
  fclose(f);

  oes_schema sc;
  CHECK(oes_schema_make(fmt, 1, E, H, I, &sc) == OES_OK, "schema: %s", oes_last_error());
  CHECK(sc.num_banks == nb, "bank count %d, schema has %d", nb, sc.num_banks);
  FILE *o = fopen(argv[2], "wb");
  CHECK(o, "cannot open %s", argv[2]);
  for (int32_t t : threads) {
    oes_cpu_moe *m = nullptr;
    CHECK(oes_cpu_moe_create(&sc, t, &m) == OES_OK, "create: %s", oes_last_error());
    for (int b = 0; b < nb; ++b)
      CHECK(oes_cpu_moe_set_source(m, b, 0, banks[b].data(), (int64_t)banks[b].size()) == OES_OK, "set_source: %s",
            oes_last_error());
    std::vector<float> y((size_t)n * H, -1.f);
    CHECK(oes_cpu_moe_run(m, 0, x.data(), ids.data(), slots.data(), w.data(), n, k, y.data()) == OES_OK, "run: %s",
          oes_last_error());
    CHECK(fwrite(y.data(), 4, y.size(), o) == y.size(), "short write");
    CHECK(oes_cpu_moe_destroy(m) == OES_OK, "destroy");
  }
  fclose(o);

  // argument errors leave no state behind
  oes_cpu_moe *m = nullptr;
  CHECK(oes_cpu_moe_create(&sc, 2, &m) == OES_OK, "create: %s", oes_last_error());
  CHECK(oes_cpu_moe_set_source(m, nb, 0, banks[0].data(), (int64_t)banks[0].size()) == OES_ERR_ARG, "bank range");
  CHECK(oes_cpu_moe_set_source(m, 0, 1, banks[0].data(), (int64_t)banks[0].size()) == OES_ERR_ARG, "layer range");
  CHECK(oes_cpu_moe_set_source(m, 0, 0, banks[0].data(), (int64_t)banks[0].size() - 1) == OES_ERR_ARG, "bank size");
  std::vector<float> y((size_t)n * H);
  // a CPU pair before every bank has a source
  CHECK(oes_cpu_moe_run(m, 0, x.data(), ids.data(), slots.data(), w.data(), n, k, y.data()) == OES_ERR_ARG,
        "run without sources");
  for (int b = 0; b < nb; ++b)
    CHECK(oes_cpu_moe_set_source(m, b, 0, banks[b].data(), (int64_t)banks[b].size()) == OES_OK, "set_source");
  std::vector<int32_t> bad = ids;
  for (size_t i = 0; i < bad.size(); ++i)
    if (slots[i] < 0) bad[i] = E;  // an id of a CPU pair outside [0, E)
  CHECK(oes_cpu_moe_run(m, 0, x.data(), bad.data(), slots.data(), w.data(), n, k, y.data()) == OES_ERR_ARG, "bad id");
  CHECK(oes_cpu_moe_run(m, 1, x.data(), ids.data(), slots.data(), w.data(), n, k, y.data()) == OES_ERR_ARG, "layer");
  CHECK(oes_cpu_moe_run(m, 0, x.data(), ids.data(), slots.data(), w.data(), n, 65, y.data()) == OES_ERR_ARG, "k");
  CHECK(oes_cpu_moe_destroy(m) == OES_OK, "destroy");
  oes_schema fp8;
  CHECK(oes_schema_make(OES_FP8_BLOCK128, 1, E, 256, 256, &fp8) == OES_OK, "fp8 schema: %s", oes_last_error());
  CHECK(oes_cpu_moe_create(&fp8, 1, &m) == OES_ERR_UNSUPPORTED && m == nullptr, "fp8 has no CPU path");
  printf("ok\n");
  return 0;
}

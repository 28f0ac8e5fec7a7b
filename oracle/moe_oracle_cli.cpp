// moe_oracle: command-line front end of the CPU oracle (TEST INFRASTRUCTURE).
//
// Reads the layer's inputs from raw little-endian files, runs oracle_forward
// on all tokens, writes the bf16 output and prints one JSON line with the
// wall time, tokens/s, fp64 GFLOP/s of the expert MLPs, threads and CPU.
// --round-y 1 rounds each slot's expert output to bf16 before the combine
// (default 0: unrounded, as the GPU path).
//
//   moe_oracle --T 64 --H 4096 --I 1024 --E 512 --K 10 --shared 1
//              [--act bf16|mxfp4] [--wfmt mxfp4|mxfp8] [--threads N] [--round-y 1|0]
//              --x x.bin --logits logits.bin [--gate gate.bin]
//              --w13 w13.bin --w13s w13s.bin --w2 w2.bin --w2s w2s.bin
//              [--out out.bin]
//
// File layouts (row-major): x bf16 [T, H]; logits float [T, E]; gate float
// [T]; w13 uint8 [E', 2I, H/2] (MXFP8: [E', 2I, H]); w13s uint8 [E', 2I, H/32];
// w2 uint8 [E', H, I/2] (MXFP8: [E', H, I]); w2s uint8 [E', H, I/32];
// out bf16 [T, H].  E' = E + shared.

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <string>
#include <vector>

#include "moe_oracle.h"

namespace {

[[noreturn]] void die(const std::string &msg) {
  std::fprintf(stderr, "moe_oracle: %s\n", msg.c_str());
  std::exit(2);
}

std::vector<uint8_t> read_file(const std::string &path, size_t want) {
  std::ifstream f(path, std::ios::binary | std::ios::ate);
  if (!f) die("cannot open " + path);
  const size_t n = static_cast<size_t>(f.tellg());
  if (n != want) die(path + ": " + std::to_string(n) + " bytes, expected " + std::to_string(want));
  std::vector<uint8_t> buf(n);
  f.seekg(0);
  f.read(reinterpret_cast<char *>(buf.data()), static_cast<std::streamsize>(n));
  return buf;
}

std::string cpu_model() {
  std::ifstream f("/proc/cpuinfo");
  std::string line;
  while (std::getline(f, line))
    if (line.rfind("model name", 0) == 0) {
      const size_t p = line.find(':');
      return p == std::string::npos ? "" : line.substr(p + 2);
    }
  return "";
}

}  // namespace

int main(int argc, char **argv) {
  std::map<std::string, std::string> arg;
  for (int i = 1; i < argc; ++i) {
    const std::string k = argv[i];
    if (k.rfind("--", 0) != 0 || i + 1 >= argc) die("bad argument " + k);
    arg[k.substr(2)] = argv[++i];
  }
  auto need = [&](const char *k) {
    if (!arg.count(k)) die(std::string("missing --") + k);
    return arg[k];
  };
  auto num = [&](const char *k) { return std::atoll(need(k).c_str()); };
  const int64_t T = num("T"), H = num("H"), I = num("I");
  const int32_t E = static_cast<int32_t>(num("E")), K = static_cast<int32_t>(num("K"));
  const int32_t shared = static_cast<int32_t>(num("shared"));
  const int act = arg.count("act") && arg["act"] == "mxfp4" ? ORACLE_ACT_MXFP4 : ORACLE_ACT_BF16;
  const int wfmt = arg.count("wfmt") && arg["wfmt"] == "mxfp8" ? ORACLE_W_MXFP8 : ORACLE_W_MXFP4;
  const int threads = arg.count("threads") ? std::atoi(arg["threads"].c_str()) : 0;
  const int round_y = arg.count("round-y") ? std::atoi(arg["round-y"].c_str()) : 0;
  if (T < 1 || H < 32 || I < 32 || E < 1 || K < 1 || K > E || (shared != 0 && shared != 1))
    die("bad shape");
  const int64_t Ep = E + shared, Kp = K + shared;
  const int64_t per = wfmt == ORACLE_W_MXFP8 ? 1 : 2;   // elements per code byte

  auto x = read_file(need("x"), T * H * 2);
  auto logits = read_file(need("logits"), T * E * 4);
  std::vector<uint8_t> gate;
  if (shared) gate = read_file(need("gate"), T * 4);
  auto w13 = read_file(need("w13"), Ep * 2 * I * H / per);
  auto w13s = read_file(need("w13s"), Ep * 2 * I * H / 32);
  auto w2 = read_file(need("w2"), Ep * H * I / per);
  auto w2s = read_file(need("w2s"), Ep * H * I / 32);

  std::vector<const uint8_t *> p13(Ep), p13s(Ep), p2(Ep), p2s(Ep);
  for (int64_t e = 0; e < Ep; ++e) {
    p13[e] = w13.data() + e * 2 * I * H / per;
    p13s[e] = w13s.data() + e * 2 * I * H / 32;
    p2[e] = w2.data() + e * H * I / per;
    p2s[e] = w2s.data() + e * H * I / 32;
  }
  std::vector<uint16_t> out(T * H);
  double seconds = 0.0;
  const int rc = oracle_forward(
      reinterpret_cast<const uint16_t *>(x.data()), reinterpret_cast<const float *>(logits.data()),
      shared ? reinterpret_cast<const float *>(gate.data()) : nullptr, p13.data(), p13s.data(),
      p2.data(), p2s.data(), T, H, I, E, K, shared, act, wfmt, 1, round_y, nullptr, 0, threads,
      nullptr,
      nullptr, out.data(), nullptr, nullptr, &seconds);
  if (rc != 0) die("oracle_forward failed with " + std::to_string(rc));
  if (arg.count("out")) {
    std::ofstream f(arg["out"], std::ios::binary);
    f.write(reinterpret_cast<const char *>(out.data()), static_cast<std::streamsize>(out.size() * 2));
    if (!f) die("cannot write " + arg["out"]);
  }
  const double flops = static_cast<double>(T * Kp) * 6.0 * static_cast<double>(H) * static_cast<double>(I);
  std::printf("{\"seconds\": %.4f, \"tokens_per_s\": %.3f, \"gflops_fp64\": %.3f, \"threads\": %d, "
              "\"cpu\": \"%s\"}\n",
              seconds, T / seconds, flops / seconds / 1e9,
              threads > 0 ? threads : oracle_default_threads(), cpu_model().c_str());
  return 0;
}

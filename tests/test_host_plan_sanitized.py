"""The C ABI's host-side planning code under AddressSanitizer and UBSan (CPU).

``api.cpp`` is compiled for the host with g++ and linked against
``host_plan_check.cpp``, which replaces the kernel launchers with checks of
the argument blocks (every byte range a kernel would touch lies inside a
buffer the caller passed, tile tables match the grid, alignment flags are
true) and the few HIP runtime calls with no-ops.  The driver then calls every
entry point on seeded random shapes with exact-size host buffers.  Planted
planning bugs in copies of ``api.cpp`` must make the check fail.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
API = os.path.join(ROOT, "collective_communication_primitives_amd", "csrc", "api.cpp")
CHECK = os.path.join(HERE, "host_plan_check.cpp")
ROCM_INCLUDE = "/opt/rocm/include"
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "collective_communication_primitives_amd", "csrc")]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _available() -> bool:
    if shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        return False
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return os.path.isabs(out) and os.path.exists(out)


pytestmark = pytest.mark.skipif(not _available(), reason="g++ with AddressSanitizer or the HIP headers missing")


@pytest.fixture(scope="module")
def check_obj(tmp_path_factory):
    obj = str(tmp_path_factory.mktemp("plan") / "host_plan_check.o")
    subprocess.run(["g++", *FLAGS, "-c", CHECK, "-o", obj], check=True, capture_output=True, text=True)
    return obj


def _build_and_run(api_source: str, check_obj: str, out_dir) -> subprocess.CompletedProcess:
    exe = str(out_dir / "plan_check")
    subprocess.run(["g++", *FLAGS, api_source, check_obj, "-o", exe], check=True, capture_output=True, text=True)
    return subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)


def test_planning_code_is_clean(check_obj, tmp_path):
    res = _build_and_run(API, check_obj, tmp_path)
    assert res.returncode == 0 and res.stdout.startswith("ok "), res.stdout[-2000:] + res.stderr[-4000:]
    assert int(res.stdout.split()[1]) > 1000  # the driver really reached the launchers


MUTANTS = {
    # the gather grid drops the partial last tile of every source
    "gather_drops_partial_tile": ("a.aligned |= 1u << k;\n            tiles += (bytes[k] + tile_bytes - 1) / tile_bytes;",
                                  "a.aligned |= 1u << k;\n            tiles += bytes[k] / tile_bytes;"),
    # a shifted fan-out piece counts its tiles without the destinations' misalignment
    "shifted_gather_tiles_short": ("tiles += dt::grid_tiles(bytes[k], md, tile_bytes);",
                                   "tiles += dt::grid_tiles(bytes[k], 0, tile_bytes);"),
    # an unaligned all-to-all block counts its tiles over its bytes, not its destination's grid
    "shifted_a2a_tiles_short": ("grid_tiles(bytes, reinterpret_cast<uintptr_t>(to) & (dt::kGridAlign - 1),",
                                "grid_tiles(bytes, 0 & (dt::kGridAlign - 1),"),

    # the windows of a large fan-out go out without their read passes
    "window_skips_read_pass": ("if (touch_first && (st = check_hip(dt::launch_gather_touch(",
                               "if (false && touch_first && (st = check_hip(dt::launch_gather_touch("),
    # in place, a large tensor is both AllReduced on its own and folded with the small ones
    "bucket_big_tensor_folded_twice": ("            if (!own(p.tensor)) pieces.push_back(piece_ref(p));",
                                       "            pieces.push_back(piece_ref(p));"),
    # the windowed fan-out of large sources skips 16 bytes after every piece
    "fan_out_window_skips_bytes": ("            off += take;\n            fill += take;",
                                   "            off += take + 16;\n            fill += take;"),
    # bucket pieces start one element late: the last piece runs past its tensor
    "bucket_piece_off_by_one": (
        "ref.ptr[r] = static_cast<char*>(grads[size_t(r) * ntensors + p.tensor]) + p.offset * es;",
        "ref.ptr[r] = static_cast<char*>(grads[size_t(r) * ntensors + p.tensor]) + (p.offset + 1) * es;"),
    # the two-shot AllReduce writes its ReduceScatter chunks one chunk too far
    "two_shot_chunk_offset": ("rs.dst[r] = static_cast<char*>(recv[r]) + r * cb;",
                              "rs.dst[r] = static_cast<char*>(recv[r]) + (r + 1) * cb;"),
    # the all-to-all never advances a column's receive offset: blocks overwrite each other
    "a2a_recv_offset_stuck": ("            recv_off[j] += bytes;\n", ""),
    # one run too many for the shard-dimension exchange
    "dims_extra_run": ("a.nruns = uint64_t(rows) * P;", "a.nruns = uint64_t(rows) * P + 1;"),
    "gather_tile_shape_mismatch": ("a.tile_bytes = uint32_t(tile_bytes);", "a.tile_bytes = uint32_t(dt::kGatherWaveTileBytes);"),
    "elems_second_range_dropped": ("            a.count2 = count - h - body;", "            a.count2 = 0;"),
    "hsdp_rs_done_never_recorded": ("    if (h->ar_stream != h->rs_stream &&\n        (st = check_hip(hipEventRecord(h->rs_done[cur_slot]",
                                    "    if (false &&\n        (st = check_hip(hipEventRecord(h->rs_done[cur_slot]"),
    "gather_split_too_wide": ("    return nranks >= 9 ? 1u : 0u;", "    return nranks >= 9 ? 3u : 0u;"),
    "dims_wave_tiles_short": ("a.tiles_per_run = uint32_t((run_bytes + dt::kDimsWaveTileBytes - 1) / dt::kDimsWaveTileBytes);",
                              "a.tiles_per_run = uint32_t(run_bytes / dt::kDimsWaveTileBytes);"),
    # every piece claimed 16-byte aligned
    "pieces_always_aligned": ("if (al) set_aligned(a, k);", "set_aligned(a, k);"),
    # the previous layer's fused buffers, whose AllReduce is still pending, may be written again
    "hsdp_fused_reuse_allowed": ("            if (h->has_prev) add_span(rd, h->prev_fused[r], h->prev_total * es, ",
                                 "            if (false) add_span(rd, h->prev_fused[r], h->prev_total * es, "),
    # a line-grid fan-out piece takes its source shift without the grid's lead
    "shifted_gather_shift_without_lead": (
        "a.lead[k] = uint32_t(md) | uint32_t((reinterpret_cast<uintptr_t>(src[k]) - md) & 15u) << 16;",
        "a.lead[k] = uint32_t(md) | uint32_t(reinterpret_cast<uintptr_t>(src[k]) & 15u) << 16;"),
    # fan-out destinations at a 16-byte boundary off their lines take the source-tiled path
    "gather_aligned_off_line": ("if (same && md == 0 && aligned16(src[k])) {",
                                "if (same && md % 16 == 0 && aligned16(src[k])) {"),
    # all-to-all blocks at a 16-byte boundary off their lines take the source-tiled path
    "a2a_aligned_off_line": ("const bool al = aligned16(from) && line_aligned(to);",
                             "const bool al = aligned16(from) && aligned16(to);"),
    # the line-grid ReduceScatter takes each chunk's grid from the inputs
    "grid_rs_lead_from_send": ("g.lead[r] = uint32_t(reinterpret_cast<uintptr_t>(out[r]) & (dt::kGridAlign - 1));",
                               "g.lead[r] = uint32_t(reinterpret_cast<uintptr_t>(send[r]) & (dt::kGridAlign - 1));"),
    # vector-aligned AllReduce inputs off their lines keep the vector two-shot form
    "allreduce_grid_ignores_input_lines": ("        lines = lines && line_aligned(send[r]);\n", "        lines = true;\n"),
    # ReduceScatter inputs off their lines keep the vector kernel
    "reduce_scatter_vec_ignores_input_lines": (
        "vec = vec && aligned16(send[r]) && aligned16(recv[r]) && line_aligned(send[r]);",
        "vec = vec && aligned16(send[r]) && aligned16(recv[r]);"),
    # ReduceScatter chunks off the lines keep the vector kernel
    "reduce_scatter_vec_ignores_chunk_lines": (
        " && (recvcount * esize_of(dtype)) % dt::kGridAlign == 0;", ";"),
    # a fan-out to destinations at offsets of their own counts its tiles over the source, not the deepest line grid
    "gather_own_offsets_source_tiles": (
        "tiles += bytes[k] ? dt::grid_tiles(bytes[k], dt::kGridAlign - 1, tile_bytes) : 0;",
        "tiles += (bytes[k] + tile_bytes - 1) / tile_bytes;"),
    # the 160 MiB line-grid threshold applied at every rank count
    "grid_two_shot_band_all_ranks": ("    if (nranks >= 6 && nranks <= 12) return ps >= (160ull << 20);",
                                     "    return ps >= (160ull << 20);"),
    # the line-grid two-shot AllReduce gives its last chunk a full chunk
    "grid_two_shot_last_chunk_full": ("            const size_t last = count - mce * size_t(nranks - 1);",
                                      "            const size_t last = mce;"),
    # only exact pointer equality is refused: a partial overlap of outputs slips through
    "overlap_check_skipped": ("    for (size_t i = 1; i < writes.size(); i++) {",
                              "    for (size_t i = writes.size(); i < writes.size(); i++) {"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_planning_bug_is_caught(check_obj, tmp_path, name):
    old, new = MUTANTS[name]
    src = open(API).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / "api_mutant.cpp"
    mutated.write_text(src.replace(old, new))
    res = _build_and_run(str(mutated), check_obj, tmp_path)
    assert res.returncode != 0, f"{name} was not caught"
